"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

The oracle follows "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3" §2.
None of these checks re-types the oracle's own formulas: each compares it
with an independent definition (textbook dense attention, a brute-force
subset search, integer arithmetic, a hand-worked example) or with an
invariant the method guarantees.
"""
import json
import math
import os

import numpy as np
import pytest

from tests.dense_reference import (bits_to_f64, dense_causal_gqa, dominance_selection, f32_to_bf16_bits,
                                   full_score_matrix, pool_by_loops)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _normal_bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _dyadic(rng, shape):
    """Integers in [-4, 4] over 4 (exact in bf16) -> (bits, integers)."""
    ints = rng.integers(-4, 5, size=shape)
    return f32_to_bf16_bits((ints / 4.0).astype(np.float32)), ints


def _problem(seed, length, hq, groups, d, di, pos=None):
    rng = _rng(seed)
    if pos is None:
        pos = np.arange(length, dtype=np.int64)
    n = len(pos)
    q_idx, q_int = _dyadic(rng, (n, groups, di))
    k_idx, k_int = _dyadic(rng, (length, di))
    q = _normal_bits(rng, (n, hq, d))
    k = _normal_bits(rng, (length, groups, d))
    v = _normal_bits(rng, (length, groups, d))
    return dict(pos=np.asarray(pos, np.int64), q_idx=q_idx, k_idx=k_idx, q=q, k=k, v=v, q_int=q_int, k_int=k_int)


# ---------------------------------------------------------------- hand-worked


def test_hand_worked_example(oracle_lib):
    """tests/golden/hand_worked_b2_k2.json: every step derived by hand."""
    with open(os.path.join(GOLDEN, "hand_worked_b2_k2.json")) as f:
        g = json.load(f)
    bs, top_k = g["block_size"], g["top_k"]
    k_idx = f32_to_bf16_bits(np.array(g["k_idx"], np.float32))
    rows = g["rows"]
    pos = np.array([r["t"] for r in rows], np.int64)
    q_idx = f32_to_bf16_bits(np.array([[r["q_idx"]] for r in rows], np.float32))
    pooled = oracle_lib.block_scores(pos, q_idx, k_idx, bs, ld=4)
    sel = oracle_lib.select(pos, pooled, bs, top_k)
    for i, r in enumerate(rows):
        c = r["t"] // bs
        np.testing.assert_array_equal(pooled[i, 0, : c + 1], np.array(r["pooled"], np.float32))
        assert np.all(np.isneginf(pooled[i, 0, c + 1:]))
        assert list(sel[i, 0]) == r["sel"]

    e = math.e
    expected_head0 = [(3 + 4 * e**2 + 7 * e) / (1 + e**2 + e),
                      (1 + 2 * e + 3 + 4 * e**2) / (2 + e + e**2),
                      3.5,
                      (1 + 7 * e) / (1 + 2 * e)]
    expected_head1 = [14 / 3, 2.5, 3.5, 8 / 3]
    q = f32_to_bf16_bits(np.tile(np.array(g["q_head_values"], np.float32)[None, :, None], (len(rows), 1, 1)))
    k = f32_to_bf16_bits(np.array(g["k"], np.float32)[:, None, None])
    v = f32_to_bf16_bits(np.array(g["v"], np.float32)[:, None, None])
    out = oracle_lib.attend(pos, q, k, v, sel, bs, scale=g["softmax_scale"])
    np.testing.assert_allclose(out[:, 0, 0], expected_head0, rtol=1e-14)
    np.testing.assert_allclose(out[:, 1, 0], expected_head1, rtol=1e-14)


# ------------------------------------------------------ steps 1-2: integers


@pytest.mark.parametrize("seed,length,bs,di,groups", [(1, 37, 4, 8, 2), (2, 300, 128, 32, 1), (3, 700, 128, 64, 3)])
def test_pooled_scores_equal_integer_arithmetic(oracle_lib, seed, length, bs, di, groups):
    """Dyadic inputs: every score is (integer dot product)/16 exactly, and the
    pooled score is the max over the block's causal tokens."""
    p = _problem(seed, length, 2, groups, 4, di)
    ld = (length - 1) // bs + 1
    pooled = oracle_lib.block_scores(p["pos"], p["q_idx"], p["k_idx"], bs, ld)
    s_int = np.einsum("ngd,ld->ngl", p["q_int"], p["k_int"])  # exact integers
    ref = pool_by_loops(s_int.astype(np.float64), p["pos"], bs, ld) / 16.0
    np.testing.assert_array_equal(pooled.astype(np.float64), ref)


def test_pooled_scores_float_inputs_match_full_matrix(oracle_lib):
    """Non-dyadic inputs: the oracle rounds the exact dot product once to
    float32; the float64 matrix product rounded to float32 agrees."""
    rng = _rng(11)
    length, di, groups, bs = 260, 64, 2, 128
    pos = np.arange(length, dtype=np.int64)
    q_idx = _normal_bits(rng, (length, groups, di))
    k_idx = _normal_bits(rng, (length, di))
    pooled = oracle_lib.block_scores(pos, q_idx, k_idx, bs, 3)
    s = full_score_matrix(bits_to_f64(q_idx), bits_to_f64(k_idx)).astype(np.float32).astype(np.float64)
    ref = pool_by_loops(s, pos, bs, 3)
    np.testing.assert_array_equal(pooled.astype(np.float64), ref)


# ---------------------------------------------------------- step 3: select


@pytest.mark.parametrize("seed", range(6))
def test_selection_equals_dominance_brute_force(oracle_lib, seed):
    """Tiny blocks (B=4) and top_k=3: the oracle's choice is the unique subset
    that dominates, found by trying every subset."""
    bs, top_k = 4, 3
    length = 41
    p = _problem(100 + seed, length, 2, 2, 4, 2)
    ld = (length - 1) // bs + 1
    pooled = oracle_lib.block_scores(p["pos"], p["q_idx"], p["k_idx"], bs, ld)
    sel = oracle_lib.select(p["pos"], pooled, bs, top_k)
    for r, t in enumerate(p["pos"]):
        c = int(t) // bs
        for g in range(2):
            want = dominance_selection(pooled[r, g], c, top_k)
            got = [int(x) for x in sel[r, g] if x >= 0]
            assert got == want, (t, g, pooled[r, g, : c + 1])


@pytest.mark.parametrize("bs,top_k,length", [(128, 16, 5000), (8, 4, 200)])
def test_selection_invariants(oracle_lib, bs, top_k, length):
    """Local block kept; min(top_k, c+1) distinct causal ids; ascending; -1 tail."""
    p = _problem(7, length, 2, 2, 4, 16)
    ld = (length - 1) // bs + 1
    pooled = oracle_lib.block_scores(p["pos"], p["q_idx"], p["k_idx"], bs, ld)
    sel = oracle_lib.select(p["pos"], pooled, bs, top_k)
    for r, t in enumerate(p["pos"]):
        c = int(t) // bs
        for g in range(2):
            row = sel[r, g]
            m = min(top_k, c + 1)
            assert np.all(row[m:] == -1)
            ids = row[:m]
            assert np.all(np.diff(ids) > 0) and ids[0] >= 0 and ids[-1] == c


def test_ties_go_to_lowest_index(oracle_lib):
    """All K_idx zero: every block scores 0, so blocks 0..14 plus the local
    block are kept.  Constant K_idx gives the same."""
    length = 3000
    for fill in (0.0, 0.5):
        k_idx = f32_to_bf16_bits(np.full((length, 8), fill, np.float32))
        q_idx = f32_to_bf16_bits(np.full((length, 2, 8), 1.0, np.float32))
        pos = np.arange(length, dtype=np.int64)
        sel = oracle_lib.select(pos, oracle_lib.block_scores(pos, q_idx, k_idx), 128, 16)
        for t in (2048, 2100, 2999):
            c = t // 128
            assert list(sel[t, 0]) == list(range(15)) + [c]


def test_planted_equal_maxima(oracle_lib):
    """Two blocks share the highest score: both are kept; when only one slot
    remains for them, the lower block wins."""
    length, bs, top_k = 64, 4, 2  # 16 blocks, one non-local slot
    k_idx = np.zeros((length, 2), np.float32)
    k_idx[4 * 9 + 1] = [1, 0]  # block 9
    k_idx[4 * 3 + 2] = [1, 0]  # block 3, same score
    pos = np.array([63], np.int64)
    q_idx = f32_to_bf16_bits(np.array([[[1.0, 0.0]]], np.float32))
    sel = oracle_lib.select(pos, oracle_lib.block_scores(pos, q_idx, f32_to_bf16_bits(k_idx), bs, 16), bs, top_k)
    assert list(sel[0, 0]) == [3, 15]
    sel3 = oracle_lib.select(pos, oracle_lib.block_scores(pos, q_idx, f32_to_bf16_bits(k_idx), bs, 16), bs, 3)
    assert list(sel3[0, 0]) == [3, 9, 15]


def test_needle_recall(oracle_lib):
    """Max-pooling: one strong token recalls its whole block, whatever the
    rest of the block holds."""
    rng = _rng(5)
    length = 8192
    for needle_block in (0, 17, 40, 62):
        k_int = rng.integers(-1, 2, size=(length, 16))
        k_int[needle_block * 128 + 77] = 4  # the needle
        q_int = np.full((1, 1, 16), 4)
        pos = np.array([length - 1], np.int64)
        pooled = oracle_lib.block_scores(pos, f32_to_bf16_bits((q_int / 4).astype(np.float32)),
                                         f32_to_bf16_bits((k_int / 4).astype(np.float32)))
        sel = oracle_lib.select(pos, pooled)
        assert needle_block in sel[0, 0]


def test_selection_scale_invariant(oracle_lib):
    """Doubling Q_idx (exact) doubles every score and changes no selection."""
    p = _problem(9, 4000, 2, 2, 4, 32)
    pooled = oracle_lib.block_scores(p["pos"], p["q_idx"], p["k_idx"])
    q2 = f32_to_bf16_bits((bits_to_f64(p["q_idx"]) * 2).astype(np.float32))
    pooled2 = oracle_lib.block_scores(p["pos"], q2, p["k_idx"])
    np.testing.assert_array_equal(pooled2[np.isfinite(pooled2)], 2 * pooled[np.isfinite(pooled)])
    np.testing.assert_array_equal(oracle_lib.select(p["pos"], pooled2), oracle_lib.select(p["pos"], pooled))


# ---------------------------------------------------------- step 4: attend


@pytest.mark.parametrize("bs,top_k,length,hq,groups,d", [(128, 16, 300, 4, 2, 16), (128, 16, 2048, 6, 2, 32),
                                                         (4, 3, 12, 4, 1, 8), (8, 4, 32, 2, 2, 8)])
def test_short_context_is_dense_attention(oracle_lib, bs, top_k, length, hq, groups, d):
    """With top_k * block_size >= context, MSA keeps every causal block and
    equals textbook dense causal GQA attention."""
    p = _problem(21, length, hq, groups, d, 16)
    _, sel, out = oracle_lib.msa(p["pos"], p["q_idx"], p["k_idx"], p["q"], p["k"], p["v"], bs, top_k)
    ref = dense_causal_gqa(bits_to_f64(p["q"]), bits_to_f64(p["k"]), bits_to_f64(p["v"]), p["pos"], 1 / math.sqrt(d))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_early_rows_of_long_context_are_dense(oracle_lib):
    """Rows t < top_k * block_size of any context attend to everything."""
    length = 2600
    p = _problem(22, length, 4, 2, 16, 16)
    pos = np.array([0, 1, 127, 128, 1000, 2047], np.int64)
    sub = {k: p[k][pos] for k in ("q", "q_idx")}
    _, sel, out = oracle_lib.msa(pos, sub["q_idx"], p["k_idx"], sub["q"], p["k"], p["v"])
    ref = dense_causal_gqa(bits_to_f64(sub["q"]), bits_to_f64(p["k"]), bits_to_f64(p["v"]), pos, 0.25)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_top_k_covering_everything_is_dense(oracle_lib):
    """top_k >= number of blocks: dense attention for every row of a long context."""
    length, bs = 900, 8
    p = _problem(23, length, 4, 2, 8, 8)
    top_k = (length - 1) // bs + 1
    _, sel, out = oracle_lib.msa(p["pos"], p["q_idx"], p["k_idx"], p["q"], p["k"], p["v"], bs, top_k)
    ref = dense_causal_gqa(bits_to_f64(p["q"]), bits_to_f64(p["k"]), bits_to_f64(p["v"]), p["pos"], 1 / math.sqrt(8))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_dense_path_equals_textbook_attention_beyond_the_cap(oracle_lib):
    """The dense path (every causal block attended) on a context longer than
    16 x 128: textbook dense causal GQA attention, and unlike MSA there."""
    length = 2600
    p = _problem(25, length, 6, 2, 16, 16)
    pos = np.array([0, 5, 127, 128, 2047, 2048, 2300, 2599], np.int64)
    q = p["q"][pos]
    out = oracle_lib.dense_attend(pos, q, p["k"], p["v"])
    ref = dense_causal_gqa(bits_to_f64(q), bits_to_f64(p["k"]), bits_to_f64(p["v"]), pos, 0.25)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    _, _, sparse = oracle_lib.msa(pos, p["q_idx"][pos], p["k_idx"], q, p["k"], p["v"])
    np.testing.assert_array_equal(sparse[:5], out[:5])  # t < 2048: identical
    assert np.abs(sparse[5:] - out[5:]).max() > 1e-3


def test_sparse_rows_equal_dense_attention_over_selected_tokens(oracle_lib):
    """Beyond 2048 tokens: each row equals textbook softmax attention over
    exactly the tokens of its selected blocks (keys and values gathered by
    index here, independently of the oracle)."""
    length = 5000
    p = _problem(24, length, 6, 2, 16, 16)
    pos = np.array([2048, 2175, 3333, 4999], np.int64)
    q_idx, q = p["q_idx"][pos], p["q"][pos]
    _, sel, out = oracle_lib.msa(pos, q_idx, p["k_idx"], q, p["k"], p["v"])
    qf, kf, vf = bits_to_f64(q), bits_to_f64(p["k"]), bits_to_f64(p["v"])
    for r, t in enumerate(pos):
        for h in range(6):
            g = h // 3
            toks = [i for b in sel[r, g] if b >= 0 for i in range(128 * b, min(128 * b + 128, t + 1))]
            assert len(toks) == 16 * 128 - (127 - t % 128)
            z = kf[toks, g] @ qf[r, h] * 0.25
            w = np.exp(z - z.max())
            np.testing.assert_allclose(out[r, h], (w / w.sum()) @ vf[toks, g], rtol=1e-12, atol=1e-13)


def test_first_token_returns_its_value(oracle_lib):
    p = _problem(25, 10, 4, 2, 16, 8)
    pos = np.array([0], np.int64)
    _, _, out = oracle_lib.msa(pos, p["q_idx"][:1], p["k_idx"], p["q"][:1], p["k"], p["v"])
    v0 = bits_to_f64(p["v"][0])
    np.testing.assert_array_equal(out[0], np.repeat(v0, 2, axis=0))


def test_output_is_convex_combination_and_order_free(oracle_lib):
    length = 4500
    p = _problem(26, length, 4, 2, 16, 16)
    pos = np.arange(2000, length, 97, dtype=np.int64)
    q_idx, q = p["q_idx"][pos], p["q"][pos]
    pooled = oracle_lib.block_scores(pos, q_idx, p["k_idx"])
    sel = oracle_lib.select(pos, pooled)
    out = oracle_lib.attend(pos, q, p["k"], p["v"], sel)
    vf = bits_to_f64(p["v"])
    for r, t in enumerate(pos):
        for g in range(2):
            toks = [i for b in sel[r, g] if b >= 0 for i in range(128 * b, min(128 * b + 128, t + 1))]
            lo, hi = vf[toks, g].min(axis=0), vf[toks, g].max(axis=0)
            for h in (2 * g, 2 * g + 1):
                assert np.all(out[r, h] >= lo - 1e-12) and np.all(out[r, h] <= hi + 1e-12)
    shuffled = sel[:, :, ::-1].copy()
    out2 = oracle_lib.attend(pos, q, p["k"], p["v"], shuffled)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)


def test_decode_row_equals_prefill_last_row(oracle_lib):
    """Rows are independent: the last row of a prefill equals a decode step
    (one query at t = N-1 over the same N cached tokens)."""
    length = 3000
    p = _problem(27, length, 4, 2, 16, 16)
    _, sel_all, out_all = oracle_lib.msa(p["pos"], p["q_idx"], p["k_idx"], p["q"], p["k"], p["v"])
    last = np.array([length - 1], np.int64)
    _, sel1, out1 = oracle_lib.msa(last, p["q_idx"][-1:], p["k_idx"], p["q"][-1:], p["k"], p["v"])
    np.testing.assert_array_equal(sel1[0], sel_all[-1])
    np.testing.assert_array_equal(out1[0], out_all[-1])


def test_invalid_selection_rejected(oracle_lib):
    p = _problem(28, 300, 2, 1, 8, 8)
    pos = np.array([200], np.int64)
    bad = np.full((1, 1, 16), -1, np.int32)
    bad[0, 0, 0] = 2  # block 2 is after the query's own block 1
    with pytest.raises(ValueError):
        oracle_lib.attend(pos, p["q"][:1], p["k"], p["v"], bad)

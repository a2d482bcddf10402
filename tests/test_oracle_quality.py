"""Pins of the oracle's selection-quality functions ("MiniMax 模型迭代与竞品分析"
§2, the paragraphs on evaluating MSA and on training the indexer): the dense
attention mass per block with coverage and recall against it, and the
indexer's target D_KL(P || Q), where P is the Main Branch's group-averaged
mass over the candidate (selected) blocks and Q the indexer's softmax over
the same blocks.

Each check compares the oracle with something other than itself: textbook
attention with block-indicator values (which makes its output exactly the
per-block mass), hand-derived closed forms, a brute-force sort for recall,
or an invariant that holds by construction.
"""
import math

import numpy as np
import pytest

from tests.dense_reference import bits_to_f64, dense_causal_gqa, f32_to_bf16_bits


def _normal_bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _mass_problem(seed, length, hq, groups, d, n_rows):
    rng = np.random.default_rng(seed)
    pos = np.sort(rng.choice(length, size=n_rows, replace=False)).astype(np.int64)
    q = _normal_bits(rng, (n_rows, hq, d))
    k = _normal_bits(rng, (length, groups, d))
    return pos, q, k


@pytest.mark.parametrize("seed,length,bs,hq,groups,d", [(0, 300, 16, 4, 2, 32), (1, 500, 8, 6, 1, 64),
                                                        (2, 129, 128, 8, 1, 16)])
def test_block_mass_is_attention_with_block_indicator_values(oracle_lib, seed, length, bs, hq, groups, d):
    """With V_i = e_{block(i)}, dense attention returns the per-block mass of each head."""
    nblk = (length + bs - 1) // bs
    assert nblk <= d
    pos, q, k = _mass_problem(seed, length, hq, groups, d, 12)
    v = np.zeros((length, groups, d))
    v[np.arange(length), :, np.arange(length) // bs] = 1.0
    scale = 1.0 / math.sqrt(d)
    heads = dense_causal_gqa(bits_to_f64(q), bits_to_f64(k), v, pos, scale)  # [n, Hq, d]
    want = heads.reshape(len(pos), groups, hq // groups, d).mean(axis=2)[:, :, :nblk]
    got = oracle_lib.block_mass(pos, q, k, bs, scale, ld=nblk)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_block_mass_sums_to_one_and_stops_at_the_local_block(oracle_lib):
    pos, q, k = _mass_problem(3, 700, 6, 2, 32, 20)
    mass = oracle_lib.block_mass(pos, q, k, 64, ld=11)
    np.testing.assert_allclose(mass.sum(axis=2), 1.0, rtol=0, atol=1e-12)
    for r, t in enumerate(pos):
        assert np.all(mass[r, :, t // 64 + 1:] == 0.0)
        assert np.all(mass[r, :, : t // 64 + 1] > 0.0)


def _random_quality_inputs(seed, n, groups, ld, bs, top_k):
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, ld * bs, size=n).astype(np.int64)
    mass = np.zeros((n, groups, ld))
    pooled = np.full((n, groups, ld), -np.inf, np.float32)
    sel = np.full((n, groups, top_k), -1, np.int32)
    for r in range(n):
        c = int(pos[r]) // bs
        for g in range(groups):
            m = rng.integers(0, 6, size=c + 1).astype(np.float64)  # small integers: plenty of ties
            m[rng.integers(0, c + 1)] += 1.0
            mass[r, g, : c + 1] = m / m.sum()
            pooled[r, g, : c + 1] = rng.standard_normal(c + 1).astype(np.float32)
            k = min(top_k, c + 1)
            sel[r, g, :k] = np.sort(rng.choice(c + 1, size=k, replace=False))
    return pos, mass, pooled, sel


def test_coverage_and_recall_against_sorting(oracle_lib):
    bs, top_k = 8, 5
    pos, mass, pooled, sel = _random_quality_inputs(4, 40, 2, 30, bs, top_k)
    cov, rec = oracle_lib.selection_quality(pos, mass, sel, bs)
    for r in range(len(pos)):
        c = int(pos[r]) // bs
        for g in range(2):
            chosen = [b for b in sel[r, g] if b >= 0]
            assert cov[r, g] == pytest.approx(sum(mass[r, g, b] for b in chosen), abs=1e-15)
            order = sorted(range(c + 1), key=lambda b: (-mass[r, g, b], b))  # larger mass first, ties to lower id
            top = set(order[: min(top_k, c + 1)])
            assert rec[r, g] == pytest.approx(len(top & set(chosen)) / len(top), abs=1e-15)


def test_all_blocks_selected_covers_everything(oracle_lib):
    bs, top_k = 16, 16
    pos, q, k = _mass_problem(5, 250, 4, 2, 32, 10)  # c + 1 <= 16 for every row
    mass = oracle_lib.block_mass(pos, q, k, bs, ld=16)
    sel = np.full((len(pos), 2, top_k), -1, np.int32)
    for r, t in enumerate(pos):
        sel[r, :, : t // bs + 1] = np.arange(t // bs + 1)
    cov, rec = oracle_lib.selection_quality(pos, mass, sel, bs)
    np.testing.assert_allclose(cov, 1.0, atol=1e-12)
    np.testing.assert_array_equal(rec, 1.0)
    # With every causal block a candidate, the Main Branch's mass is the dense mass.
    sel_mass = oracle_lib.selected_mass(pos, q, k, sel, bs, ld=16)
    np.testing.assert_allclose(sel_mass, mass, rtol=0, atol=1e-12)


def _bits(values):
    return f32_to_bf16_bits(np.asarray(values, np.float32))


def _hand_mass_case():
    """Block size 2, one KV group of two heads, head_dim 1, query at t = 4 (local block 2
    holds token 4 only; token 5 exists but lies after the query).  Keys k = (1, 1, 1, 0, 1, 1),
    scale ln 3, so a key of 1 weighs 3 and a key of 0 weighs 1 under head 0 (q = 1), while head 1
    (q = 0) weighs every token 1.  Selected blocks {1, 2}: tokens 2, 3, 4.
      head 0: weights 3, 1, 3 -> block 1: 4/7, block 2: 3/7
      head 1: weights 1, 1, 1 -> block 1: 2/3, block 2: 1/3
      P (average): block 1: 13/21, block 2: 8/21, block 0: 0."""
    pos = np.array([4], np.int64)
    q = _bits([[[1.0], [0.0]]])                          # [n=1, Hq=2, D=1]
    k = _bits([[[1.0]], [[1.0]], [[1.0]], [[0.0]], [[1.0]], [[1.0]]])  # [L=6, G=1, D=1]
    sel = np.array([[[1, 2]]], np.int32)
    return pos, q, k, sel


def test_selected_mass_hand_example(oracle_lib):
    pos, q, k, sel = _hand_mass_case()
    got = oracle_lib.selected_mass(pos, q, k, sel, block_size=2, scale=math.log(3.0), ld=3)
    np.testing.assert_allclose(got[0, 0], [0.0, 13 / 21, 8 / 21], rtol=0, atol=1e-14)


def test_kl_hand_example(oracle_lib):
    """P of the hand-worked mass case, indexer scores S = (5, 1, 0) on blocks 0..2 with
    blocks {1, 2} selected: Q over the candidates only, Q = (e, 1) / (1 + e); block 0 is not
    a candidate, so its large score does not enter Q.
      D_KL = 13/21 ln(13/21 (1 + e) / e) + 8/21 ln(8/21 (1 + e))."""
    pos, q, k, sel = _hand_mass_case()
    p = oracle_lib.selected_mass(pos, q, k, sel, block_size=2, scale=math.log(3.0), ld=3)
    pooled = np.array([[[5.0, 1.0, 0.0]]], np.float32)
    kl = oracle_lib.indexer_kl(pos, p, pooled, sel, block_size=2)
    e = math.e
    want = 13 / 21 * math.log(13 / 21 * (1 + e) / e) + 8 / 21 * math.log(8 / 21 * (1 + e))
    assert kl[0, 0] == pytest.approx(want, abs=1e-7)
    # P = (3/4, 1/4) on candidates {0, 2} against Q = (1/4, 3/4) from scores (0, ln 3):
    # D_KL = 3/4 ln 3 + 1/4 ln(1/3) = (1/2) ln 3, whatever the score of block 1.
    p2 = np.array([[[0.75, 0.0, 0.25]]])
    s2 = np.array([[[0.0, 100.0, math.log(3.0)]]], np.float32)
    kl2 = oracle_lib.indexer_kl(np.array([5], np.int64), p2, s2, np.array([[[0, 2]]], np.int32), block_size=2)
    assert kl2[0, 0] == pytest.approx(0.5 * math.log(3.0), abs=1e-7)


def _numpy_selected_mass(pos, q, k, sel, bs, scale, ld):
    """Textbook softmax attention over the selected tokens with V_i = e_{block(i)}, averaged
    over each group's heads: exactly the Main Branch's mass per selected block."""
    qf, kf = bits_to_f64(q), bits_to_f64(k)
    n, hq, _ = qf.shape
    groups = kf.shape[1]
    gs = hq // groups
    out = np.zeros((n, groups, ld))
    for r, t in enumerate(pos):
        for g in range(groups):
            tok = np.concatenate([np.arange(b * bs, min(b * bs + bs, t + 1)) for b in sel[r, g] if b >= 0])
            onehot = np.zeros((len(tok), ld))
            onehot[np.arange(len(tok)), tok // bs] = 1.0
            for j in range(gs):
                z = scale * (kf[tok, g] @ qf[r, g * gs + j])
                p = np.exp(z - z.max())
                out[r, g] += (p / p.sum()) @ onehot / gs
    return out


@pytest.mark.parametrize("seed,length,bs,top_k,hq,groups,d", [(7, 700, 16, 5, 6, 2, 32), (8, 900, 32, 4, 4, 1, 64)])
def test_selected_mass_is_attention_over_the_selection(oracle_lib, seed, length, bs, top_k, hq, groups, d):
    """Against textbook attention over the selected tokens; each row sums to 1 over its
    candidates, and blocks that are not selected get no mass."""
    pos, q, k = _mass_problem(seed, length, hq, groups, d, 14)
    rng = np.random.default_rng(seed)
    ld = (length + bs - 1) // bs
    sel = np.full((len(pos), groups, top_k), -1, np.int32)
    for r, t in enumerate(pos):
        c = int(t) // bs
        for g in range(groups):
            pick = rng.choice(c, size=min(top_k - 1, c), replace=False) if c else np.array([], np.int64)
            chosen = np.sort(np.append(pick, c))
            sel[r, g, : len(chosen)] = chosen
    scale = 1.0 / math.sqrt(d)
    got = oracle_lib.selected_mass(pos, q, k, sel, bs, scale, ld=ld)
    want = _numpy_selected_mass(pos, q, k, sel, bs, scale, ld)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got.sum(axis=2), 1.0, rtol=0, atol=1e-12)
    for r in range(len(pos)):
        for g in range(groups):
            off = np.setdiff1d(np.arange(ld), sel[r, g][sel[r, g] >= 0])
            assert np.all(got[r, g, off] == 0.0)


def test_kl_vanishes_when_the_indexer_matches_and_is_nonnegative(oracle_lib):
    bs, top_k = 8, 5
    pos, mass, pooled, sel = _random_quality_inputs(6, 30, 2, 25, bs, top_k)
    # P over each row's candidates: the random masses restricted to the selection, renormalised.
    p = np.zeros_like(mass)
    for r in range(len(pos)):
        for g in range(2):
            chosen = sel[r, g][sel[r, g] >= 0]
            p[r, g, chosen] = mass[r, g, chosen] + 0.25
            p[r, g] /= p[r, g].sum()
    kl = oracle_lib.indexer_kl(pos, p, pooled, sel, bs)
    assert np.all(kl >= -1e-12)  # Gibbs' inequality
    matched = np.where(p > 0, np.log(np.where(p > 0, p, 1.0)), 50.0).astype(np.float32)  # non-candidates: any score
    kl0 = oracle_lib.indexer_kl(pos, p, matched, sel, bs)
    np.testing.assert_allclose(kl0, 0.0, atol=2e-6)

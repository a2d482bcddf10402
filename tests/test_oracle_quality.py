"""Pins of the oracle's selection-quality functions (dense attention mass per
block, coverage, recall, D_KL(P || Q); "MiniMax 模型迭代与竞品分析" §2, the
paragraphs on indexer training and on evaluating MSA).

Each check compares the oracle with something other than itself: textbook
dense attention with block-indicator values (which makes its output exactly
the per-block mass), a hand-derived KL value, a brute-force sort for recall,
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
    cov, rec, _ = oracle_lib.selection_quality(pos, mass, pooled, sel, bs)
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
    pooled = np.zeros(mass.shape, np.float32)
    cov, rec, kl = oracle_lib.selection_quality(pos, mass, pooled, sel, bs)
    np.testing.assert_allclose(cov, 1.0, atol=1e-12)
    np.testing.assert_array_equal(rec, 1.0)
    assert np.all(kl >= -1e-12)


def test_kl_hand_example(oracle_lib):
    """P = (3/4, 1/4), indexer scores (0, ln 3) so Q = (1/4, 3/4):
    D_KL = 3/4 ln 3 + 1/4 ln(1/3) = (1/2) ln 3."""
    pos = np.array([5], np.int64)  # block size 4: blocks 0 and 1
    mass = np.array([[[0.75, 0.25]]])
    pooled = np.array([[[0.0, math.log(3.0)]]], np.float32)
    sel = np.array([[[0, 1]]], np.int32)
    cov, rec, kl = oracle_lib.selection_quality(pos, mass, pooled, sel, 4)
    assert kl[0, 0] == pytest.approx(0.5 * math.log(3.0), abs=1e-7)
    assert cov[0, 0] == 1.0 and rec[0, 0] == 1.0


def test_kl_vanishes_when_the_indexer_matches_and_is_nonnegative(oracle_lib):
    bs, top_k = 8, 5
    pos, mass, pooled, sel = _random_quality_inputs(6, 30, 2, 25, bs, top_k)
    _, _, kl = oracle_lib.selection_quality(pos, mass, pooled, sel, bs)
    assert np.all(kl >= -1e-12)  # Gibbs' inequality
    matched = np.where(mass > 0, np.log(np.where(mass > 0, mass, 1.0)), -np.inf).astype(np.float32)
    matched[mass == 0] = -1e30  # empty blocks: Q ~ 0 where P = 0
    _, _, kl0 = oracle_lib.selection_quality(pos, mass, matched, sel, bs)
    np.testing.assert_allclose(kl0, 0.0, atol=2e-6)

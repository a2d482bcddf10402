"""Pins of oracle.scores_matmul, the matrix-product form of MSA steps 1-2
("MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2: score every causal
key against the shared K_idx, max-pool per 128-token block) that the
full-size parity tests use to check every row of a long prefill.

It must equal exact integer arithmetic and, bit for bit, the C oracle's
loop, for every batching of the rows; and it must refuse inputs for which a
float32 matrix product would not be exact.
"""
import numpy as np
import pytest

from oracle import scores_matmul
from tests.dense_reference import f32_to_bf16_bits, pool_by_loops


def _dyadic(rng, shape):
    ints = rng.integers(-4, 5, size=shape)
    return f32_to_bf16_bits((ints / 4.0).astype(np.float32)), ints


@pytest.mark.parametrize("seed,length,first,bs,di,groups,rpb", [
    (1, 37, 0, 4, 8, 2, 5),          # tiny blocks, batches not aligned to blocks
    (2, 700, 300, 128, 64, 3, 128),  # a chunk starting mid-block
    (3, 1000, 999, 128, 32, 1, 64),  # one row
    (4, 2600, 0, 128, 64, 8, 512),   # many blocks, a batch spanning several blocks
])
def test_equals_integer_arithmetic(seed, length, first, bs, di, groups, rpb):
    rng = np.random.default_rng(seed)
    pos = np.arange(first, length, dtype=np.int64)
    q_bits, q_int = _dyadic(rng, (len(pos), groups, di))
    k_bits, k_int = _dyadic(rng, (length, di))
    ld = (length - 1) // bs + 1
    got = scores_matmul.block_scores(first, q_bits, k_bits, bs, ld, rows_per_batch=rpb)
    s_int = np.einsum("ngd,ld->ngl", q_int, k_int)  # exact integers
    want = pool_by_loops(s_int.astype(np.float64), pos, bs, ld) / 16.0
    np.testing.assert_array_equal(got.astype(np.float64), want)
    assert not np.any(np.signbit(got) & (got == 0)), "-0 must be written as +0"


@pytest.mark.parametrize("first,rpb", [(0, 512), (1500, 100), (4000, 7)])
def test_equals_the_c_loop_bit_for_bit(oracle_lib, first, rpb):
    rng = np.random.default_rng(5)
    length, di, groups = 4100, 64, 4
    pos = np.arange(first, length, dtype=np.int64)
    q_bits, _ = _dyadic(rng, (len(pos), groups, di))
    k_bits, _ = _dyadic(rng, (length + 50, di))  # keys after the last row are never scored
    ld = 40
    want = oracle_lib.block_scores(pos, q_bits, k_bits, 128, ld)
    got = scores_matmul.block_scores(first, q_bits, k_bits, 128, ld, rows_per_batch=rpb)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_refuses_inputs_a_float32_product_would_round():
    rng = np.random.default_rng(6)
    q = f32_to_bf16_bits(rng.standard_normal((10, 2, 64)).astype(np.float32))  # not dyadic at small exponents
    k, _ = _dyadic(rng, (20, 64))
    with pytest.raises(ValueError):
        scores_matmul.block_scores(10, q, k, 128)
    wide = f32_to_bf16_bits(np.full((10, 2, 64), 1024.0, np.float32))  # dyadic, but sums reach 2^24
    kw = f32_to_bf16_bits(np.full((20, 64), 256.0, np.float32))  # 64 * 1024 * 256 = 2^24
    with pytest.raises(ValueError):
        scores_matmul.block_scores(10, wide, kw, 128)

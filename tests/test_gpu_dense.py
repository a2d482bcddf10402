"""Parity of the dense causal attention call (msa_dense_attn_prefill) with the
oracle's dense path (every causal block attended), through the C ABI.

Outputs must be within max-abs 2e-2 and mean-abs 2e-3 of the oracle's
double-precision result, the tolerance of the Main Branch.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_score_amd import ops
from block_sparse_long_score_amd.inputs import WORKLOADS, bf16_bits, make_inputs
from block_sparse_long_score_amd.pipeline import MsaRunner
from tests.gpu_helpers import MAX_ABS, MEAN_ABS, seq_rows

pytestmark = pytest.mark.gpu

M2 = WORKLOADS["c1"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _dense(w):
    _announce(f"dense {w.name}: seq_lens={w.seq_lens[:4]}{'...' if w.num_seqs > 4 else ''} q_lens={w.q_lens[:4]} "
              f"Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim}")
    runner = MsaRunner(make_inputs(w, "cuda"))
    runner.append()
    out = torch.full_like(runner.inputs.q, float("nan"))
    ops.msa_dense_attn_prefill(runner.dims, runner.cache, runner.batch, runner.inputs.q, out)
    torch.cuda.synchronize()
    return runner, out


def _oracle_dense(inp, s, positions):
    positions = np.asarray(positions, dtype=np.int64)
    rows = torch.from_numpy(seq_rows(inp, s, positions)).to(inp.q.device)
    off = int(inp.tok_off[s])
    length = int(positions.max()) + 1
    k = bf16_bits(inp.k[off:off + length])
    v = bf16_bits(inp.v[off:off + length])
    q = bf16_bits(inp.q.index_select(0, rows))
    return rows, oracle.dense_attend(positions, q, k, v, inp.workload.block_size)


def _compare(runner, out, s, positions):
    inp = runner.inputs
    rows, want = _oracle_dense(inp, s, positions)
    got = out.index_select(0, rows).float().cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), "rows left unwritten"
    max_abs, mean_abs = float(err.max()), float(err.mean())
    assert max_abs <= MAX_ABS and mean_abs <= MEAN_ABS, (s, max_abs, mean_abs)


def _all_rows(runner, out):
    w = runner.inputs.workload
    for s in range(w.num_seqs):
        if w.q_lens[s]:
            _compare(runner, out, s, runner.inputs.positions(s))


def test_dense_c0_all_rows():
    """One KV group (8 heads, D = 64): every XCD deals tiles of the same group."""
    runner, out = _dense(WORKLOADS["c0"])
    _all_rows(runner, out)


def test_dense_ragged_prefill_beyond_the_cap():
    """3001 rows: a partial first tile and rows past 16 x 128, where dense differs from MSA."""
    runner, out = _dense(M2.with_sizes("dense_ragged", [3001], [3001]))
    _all_rows(runner, out)


def test_dense_chunk_starting_mid_block():
    runner, out = _dense(M2.with_sizes("dense_chunk", [5000], [777]))
    _all_rows(runner, out)


def test_dense_multi_sequence_batch_permuted_table():
    runner, out = _dense(M2.with_sizes("dense_multi", [2500, 129, 1, 4100, 2048], [2500, 60, 1, 900, 17],
                                       permuted_table=True))
    _all_rows(runner, out)
    assert torch.isfinite(out.float()).all()


def test_dense_one_query_per_sequence():
    runner, out = _dense(M2.with_sizes("dense_decode", [1, 128, 129, 2049, 5000, 9999], [1] * 6,
                                       permuted_table=True))
    _all_rows(runner, out)


def test_dense_m3_shape():
    """64 query heads over 4 KV heads (two XCDs per group)."""
    runner, out = _dense(WORKLOADS["m3p"].with_sizes("dense_m3", [2600], [2600]))
    _all_rows(runner, out)


def test_dense_matches_msa_below_the_cap():
    """Rows before position 2048 attend to every causal block under MSA too."""
    w = M2.with_sizes("dense_vs_msa", [2048], [2048])
    runner, out = _dense(w)
    runner.step()
    torch.cuda.synchronize()
    diff = (runner.out.float() - out.float()).abs()
    assert float(diff.max()) <= 2 * MAX_ABS and float(diff.mean()) <= MEAN_ABS


def test_dense_c1_full_size_sampled_rows():
    runner, out = _dense(WORKLOADS["c1"])
    rng = np.random.default_rng(11)
    pos = np.unique(np.concatenate([[0, 127, 128, 2047, 2048, 32767], rng.integers(0, 32768, 90)]))
    _compare(runner, out, 0, pos)
    assert torch.isfinite(out.float()).all()


def test_dense_c3_full_size_sampled_rows():
    runner, out = _dense(WORKLOADS["c3"])
    rng = np.random.default_rng(12)
    pos = np.unique(np.concatenate([[0, 128, 65535, 131071], rng.integers(0, 131072, 20)]))
    _compare(runner, out, 0, pos)
    assert torch.isfinite(out.float()).all()


def _dense_decode(w):
    _announce(f"dense decode {w.name}: seq_lens={w.seq_lens[:4]}{'...' if w.num_seqs > 4 else ''} "
              f"Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim}")
    runner = MsaRunner(make_inputs(w, "cuda"))
    runner.append()
    out = torch.full_like(runner.inputs.q, float("nan"))
    need = ops.msa_workspace_size(runner.dims, runner.cache, runner.batch, ops.MSA_CALL_DENSE_ATTN_DECODE)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ops.msa_dense_attn_decode(runner.dims, runner.cache, runner.batch, runner.inputs.q, out, ws)
    torch.cuda.synchronize()
    return runner, out


def test_dense_decode_ragged_lengths_permuted_table():
    """Contexts from one token to past several 64-block splits, on a scattered block table."""
    w = M2.with_sizes("dense_dec", [1, 128, 129, 2049, 5000, 9999, 8192, 8193, 8320], [1] * 9, permuted_table=True)
    runner, out = _dense_decode(w)
    _all_rows(runner, out)


def test_dense_decode_group_sizes():
    for name, w in (("g16", WORKLOADS["m3d"].with_sizes("dense_dec_g16", [3000, 9001], [1, 1])),
                    ("g8_d64", WORKLOADS["c0"].with_sizes("dense_dec_g8", [4096, 777, 8500], [1, 1, 1]))):
        runner, out = _dense_decode(w)
        _all_rows(runner, out)


def test_dense_decode_equals_dense_prefill_kernel():
    """Both dense calls on the same one-query batch."""
    w = M2.with_sizes("dense_dec_eq", [700, 4097, 20000], [1, 1, 1], permuted_table=True)
    runner, out = _dense_decode(w)
    ref = torch.full_like(out, float("nan"))
    ops.msa_dense_attn_prefill(runner.dims, runner.cache, runner.batch, runner.inputs.q, ref)
    torch.cuda.synchronize()
    diff = (out.float() - ref.float()).abs()
    assert float(diff.max()) <= 2 * MAX_ABS and float(diff.mean()) <= MEAN_ABS


def test_dense_decode_c2_full_size_sampled_sequences():
    runner, out = _dense_decode(WORKLOADS["c2"])
    for s in (0, 13, 31):
        _compare(runner, out, s, [131071])
    assert torch.isfinite(out.float()).all()


def test_dense_decode_c4d_1m_one_sequence():
    runner, out = _dense_decode(WORKLOADS["c4d"])
    _compare(runner, out, 2, [(1 << 20) - 1])
    assert torch.isfinite(out.float()).all()


def _oracle_dense_without(inp, s, positions, absent):
    """Dense attention over every causal block except the `absent` ones."""
    positions = np.asarray(positions, dtype=np.int64)
    rows = torch.from_numpy(seq_rows(inp, s, positions)).to(inp.q.device)
    off = int(inp.tok_off[s])
    length = int(positions.max()) + 1
    k = bf16_bits(inp.k[off:off + length])
    v = bf16_bits(inp.v[off:off + length])
    q = bf16_bits(inp.q.index_select(0, rows))
    w = inp.workload
    nblk = (length + 127) // 128
    sel = np.full((len(positions), w.num_kv_heads, nblk), -1, dtype=np.int32)
    for r, t in enumerate(positions):
        keep = [b for b in range(int(t) // 128 + 1) if b not in absent]
        sel[r, :, :len(keep)] = keep
    return rows, oracle.attend(positions, q, k, v, sel, w.block_size)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_dense_blocks_outside_the_cache_hold_no_keys(mode):
    """Block-table entries outside [0, num_blocks) are skipped, as in the sparse calls."""
    q_len = 700 if mode == "prefill" else 1
    w = M2.with_sizes(f"dense_absent_{mode}", [3000], [q_len], permuted_table=True)
    runner = MsaRunner(make_inputs(w, "cuda"))
    runner.append()
    absent = {3: -1, 7: runner.cache.k.shape[0], 10: -5}
    for b, v in absent.items():
        runner.cache.block_table[0, b] = v
    out = torch.full_like(runner.inputs.q, float("nan"))
    if mode == "prefill":
        ops.msa_dense_attn_prefill(runner.dims, runner.cache, runner.batch, runner.inputs.q, out)
    else:
        need = ops.msa_workspace_size(runner.dims, runner.cache, runner.batch, ops.MSA_CALL_DENSE_ATTN_DECODE)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ops.msa_dense_attn_decode(runner.dims, runner.cache, runner.batch, runner.inputs.q, out, ws)
    torch.cuda.synchronize()
    pos = runner.inputs.positions(0)
    rows, want = _oracle_dense_without(runner.inputs, 0, pos, set(absent))
    got = out.index_select(0, rows).float().cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    assert float(err.max()) <= MAX_ABS and float(err.mean()) <= MEAN_ABS


def test_dense_batch_with_sequences_without_queries():
    """Sequences with no query rows this step take no part (and write nothing)."""
    w = M2.with_sizes("dense_noq", [2000, 500, 4200, 129], [0, 300, 0, 129], permuted_table=True)
    runner, out = _dense(w)
    _all_rows(runner, out)
    assert torch.isfinite(out.float()).all()

"""Helpers for the GPU parity tests: run the oracle on chosen rows of a
workload and compare with what the HIP path produced.

The oracle reads only the synthetic inputs (never a GPU result): index keys
up to the row's position, and the K/V tokens of the blocks the oracle itself
selected.  Unselected tokens are filled with NaN on the host, so an oracle
that touched them would produce NaN and fail the comparison.
"""
import numpy as np
import torch

import oracle
from block_sparse_long_score_amd.inputs import bf16_bits
from oracle import scores_matmul

MAX_ABS = 2e-2   # spec tolerance on attention outputs (bf16 in, fp32 accumulate)
MEAN_ABS = 2e-3
BF16_NAN = 0x7FC0


def seq_rows(inp, s, positions):
    """Query-row indices of absolute positions of sequence s."""
    w = inp.workload
    first = w.seq_lens[s] - w.q_lens[s]
    positions = np.asarray(positions, dtype=np.int64)
    assert np.all((positions >= first) & (positions < w.seq_lens[s]))
    return inp.cu_q[s] + (positions - first)


def oracle_rows(inp, s, positions, attend=True):
    """(pooled, sel, out) of the oracle for some query rows of sequence s."""
    w = inp.workload
    positions = np.asarray(positions, dtype=np.int64)
    rows = torch.from_numpy(seq_rows(inp, s, positions)).to(inp.q.device)
    off = int(inp.tok_off[s])
    length = int(positions.max()) + 1
    k_idx = bf16_bits(inp.k_idx[off:off + length])
    q_idx = bf16_bits(inp.q_idx.index_select(0, rows))
    ld = (w.seq_lens[s] + 127) // 128
    pooled = oracle.block_scores(positions, q_idx, k_idx, w.block_size, ld)
    sel = oracle.select(positions, pooled, w.block_size, w.top_k)
    if not attend:
        return pooled, sel, None
    blocks = np.unique(sel[sel >= 0]).astype(np.int64)
    tok = (blocks[:, None] * w.block_size + np.arange(w.block_size)[None, :]).ravel()
    tok = tok[tok < length]
    shape = (length, w.num_kv_heads, w.head_dim)
    k_host = np.full(shape, BF16_NAN, np.uint16)
    v_host = np.full(shape, BF16_NAN, np.uint16)
    tok_dev = torch.from_numpy(tok + off).to(inp.k.device)
    k_host[tok] = bf16_bits(inp.k.index_select(0, tok_dev))
    v_host[tok] = bf16_bits(inp.v.index_select(0, tok_dev))
    q = bf16_bits(inp.q.index_select(0, rows))
    out = oracle.attend(positions, q, k_host, v_host, sel, w.block_size)
    return pooled, sel, out


def compare_rows(runner, s, positions, check_scores=True, check_out=True):
    """Compare the HIP results of runner (after a step) with the oracle on
    rows of sequence s.  Returns (max_abs, mean_abs) of the outputs."""
    inp = runner.inputs
    positions = np.asarray(positions, dtype=np.int64)
    pooled, sel, out = oracle_rows(inp, s, positions, attend=check_out)
    rows = torch.from_numpy(seq_rows(inp, s, positions)).to(inp.q.device)
    gpu_sel = runner.sel.index_select(0, rows).cpu().numpy()
    bad = np.argwhere(np.any(gpu_sel != sel, axis=-1))
    assert bad.size == 0, (f"selection mismatch at {len(bad)} (row, group) pairs, first: position "
                           f"{positions[bad[0][0]]} group {bad[0][1]}: gpu {gpu_sel[tuple(bad[0])]} "
                           f"oracle {sel[tuple(bad[0])]}")
    if check_scores:
        gpu_scores = runner.scores.index_select(0, rows).cpu().numpy()
        for i, t in enumerate(positions):
            c = int(t) // 128
            np.testing.assert_array_equal(gpu_scores[i, :, :c + 1], pooled[i, :, :c + 1],
                                          err_msg=f"pooled scores differ at position {t}")
    if not check_out:
        return None
    gpu_out = runner.out.index_select(0, rows).float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(out)), "oracle touched a token outside its selection"
    err = np.abs(gpu_out - out)
    max_abs, mean_abs = float(err.max()), float(err.mean())
    assert max_abs <= MAX_ABS and mean_abs <= MEAN_ABS, (max_abs, mean_abs)
    return max_abs, mean_abs


def check_selection_invariants(runner):
    """Properties of every row's selection that hold at any size."""
    w = runner.inputs.workload
    sel = runner.sel.cpu().numpy()
    pos = np.concatenate([runner.inputs.positions(s) for s in range(w.num_seqs)])
    c = pos // 128
    nsel = np.minimum(w.top_k, c + 1)
    valid = np.arange(w.top_k)[None, None, :] < nsel[:, None, None]
    assert np.all(sel[~np.broadcast_to(valid, sel.shape)] == -1)
    last = np.take_along_axis(sel, (nsel - 1)[:, None, None].repeat(sel.shape[1], 1), axis=2)[..., 0]
    assert np.all(last == c[:, None]), "local block missing or not last"
    d = np.diff(sel, axis=2)
    assert np.all((d > 0) | ~np.broadcast_to(valid[:, :, 1:], d.shape)), "not strictly ascending"
    assert np.all((sel >= 0) | ~np.broadcast_to(valid, sel.shape))


def compare_row_range(runner, s, r0, r1, check_out=True, batch=2048):
    """Every query row of sequence s with row index (within the sequence) in
    [r0, r1) against the oracle, in batches: pooled scores bit for bit (steps
    1-2 by the pinned matrix-product form of the oracle), selections bit for
    bit (the oracle's select on the oracle's scores), and, with check_out,
    the outputs within the tolerance (the oracle's attention over all of the
    sequence's keys).  Returns (max_abs, mean_abs) over the range, or None."""
    inp = runner.inputs
    w = inp.workload
    first = w.seq_lens[s] - w.q_lens[s]
    off = int(inp.tok_off[s])
    last_pos = first + r1 - 1
    k_idx = bf16_bits(inp.k_idx[off:off + last_pos + 1])
    if check_out:
        k = bf16_bits(inp.k[off:off + last_pos + 1])
        v = bf16_bits(inp.v[off:off + last_pos + 1])
    ld = runner.ld
    worst, total, count = 0.0, 0.0, 0
    for b0 in range(r0, r1, batch):
        b1 = min(r1, b0 + batch)
        pos = np.arange(first + b0, first + b1, dtype=np.int64)
        rows = torch.arange(int(inp.cu_q[s]) + b0, int(inp.cu_q[s]) + b1, device=inp.q.device)
        q_idx = bf16_bits(inp.q_idx.index_select(0, rows))
        pooled = scores_matmul.block_scores(int(pos[0]), q_idx, k_idx, w.block_size, ld)
        gpu_scores = runner.scores.index_select(0, rows).cpu().numpy()
        c = pos // w.block_size
        causal = np.arange(ld)[None, None, :] <= c[:, None, None]
        bad = np.argwhere(causal & (gpu_scores.view(np.uint32) != pooled.view(np.uint32)))
        assert bad.size == 0, (f"pooled scores differ at {len(bad)} entries, first: position {pos[bad[0][0]]} "
                               f"group {bad[0][1]} block {bad[0][2]}")
        sel = oracle.select(pos, pooled, w.block_size, w.top_k)
        gpu_sel = runner.sel.index_select(0, rows).cpu().numpy()
        bad = np.argwhere(np.any(gpu_sel != sel, axis=-1))
        assert bad.size == 0, (f"selection mismatch at {len(bad)} (row, group) pairs, first: position "
                               f"{pos[bad[0][0]]} group {bad[0][1]}: gpu {gpu_sel[tuple(bad[0])]} "
                               f"oracle {sel[tuple(bad[0])]}")
        if not check_out:
            continue
        out = oracle.attend(pos, bf16_bits(inp.q.index_select(0, rows)), k, v, sel, w.block_size)
        err = np.abs(runner.out.index_select(0, rows).float().cpu().numpy().astype(np.float64) - out)
        worst = max(worst, float(err.max()))
        total += float(err.sum())
        count += err.size
    if not check_out:
        return None
    max_abs, mean_abs = worst, total / count
    assert max_abs <= MAX_ABS and mean_abs <= MEAN_ABS, (max_abs, mean_abs)
    return max_abs, mean_abs

"""msa_index_select (scoring, pooling and top-k in one call, chunked through
the workspace) against the two separate calls: selections must be identical,
with the suggested workspace and with small ones that force many chunks
(row ranges of one long sequence, and runs of whole sequences)."""
import sys

import pytest
import torch

import numpy as np

from block_sparse_long_score_amd import ops
from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs
from block_sparse_long_score_amd.pipeline import MsaRunner
from tests.gpu_helpers import check_selection_invariants, oracle_rows, seq_rows

pytestmark = pytest.mark.gpu

M2 = WORKLOADS["c1"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _select(runner, rows_per_chunk=None):
    """sel from msa_index_select; rows_per_chunk sizes the workspace (None: the suggested size)."""
    w = runner.inputs.workload
    if rows_per_chunk is None:
        nbytes = ops.msa_workspace_size(runner.dims, runner.cache, runner.batch, ops.MSA_CALL_INDEX_SELECT)
    else:
        nbytes = 256 + rows_per_chunk * w.num_kv_heads * runner.ld * 4
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sel = torch.full_like(runner.sel, 0x7777)
    ops.msa_index_select(runner.dims, runner.cache, runner.batch, runner.inputs.q_idx, sel, ws)
    torch.cuda.synchronize()
    return sel


CASES = {
    "c0": WORKLOADS["c0"],
    "ragged": M2.with_sizes("sel_ragged", [3001], [3001]),
    "chunk_mid_block": M2.with_sizes("sel_chunk", [5000], [777]),
    "multi_seq": M2.with_sizes("sel_multi", [2500, 129, 1, 4100, 2048], [2500, 60, 1, 900, 17], permuted_table=True),
    "decode": M2.with_sizes("sel_decode", [1, 128, 129, 2049, 5000, 9999, 2048, 2049], [1] * 8, permuted_table=True),
    "with_empty_seqs": M2.with_sizes("sel_empty", [2000, 500, 4200, 129], [0, 300, 0, 129], permuted_table=True),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("rows_per_chunk", [None, 37, 1])
def test_index_select_equals_score_then_topk(name, rows_per_chunk):
    w = CASES[name]
    if rows_per_chunk == 1 and w.total_q > 1000:
        rows_per_chunk = 257  # one row per chunk only on the small batches (thousands of launches otherwise)
    _announce(f"select {name} rows_per_chunk={rows_per_chunk}")
    runner = MsaRunner(make_inputs(w, "cuda"))
    runner.step()
    sel = _select(runner, rows_per_chunk)
    assert torch.equal(sel, runner.sel)


def _sampled_positions(w, s, count, seed):
    first, n = w.seq_lens[s] - w.q_lens[s], w.seq_lens[s]
    rng = np.random.default_rng(seed)
    fixed = [p for p in (first, 2047, 2048, n - 1) if first <= p < n]
    return np.unique(np.concatenate([fixed, rng.integers(first, n, size=count)]).astype(np.int64))


@pytest.mark.parametrize("wl", ["c3", "c4p", "c2"])
def test_index_select_full_size(wl):
    """msa_index_select at full size: equal to the two calls on every row, and to
    the oracle on sampled rows of every sequence."""
    _announce(f"select full size {wl}")
    w = WORKLOADS[wl]
    runner = MsaRunner(make_inputs(w, "cuda"), chunk_rows=16384)
    runner.step()
    sel = _select(runner)
    assert torch.equal(sel, runner.sel)
    check_selection_invariants(runner)
    for s in range(w.num_seqs):
        pos = _sampled_positions(w, s, 128 if w.q_lens[s] > 1 else 0, 7 + s)
        _, want, _ = oracle_rows(runner.inputs, s, pos, attend=False)
        rows = torch.from_numpy(seq_rows(runner.inputs, s, pos)).to(sel.device)
        got = sel.index_select(0, rows).cpu().numpy()
        np.testing.assert_array_equal(got, want, err_msg=f"{wl} sequence {s}: msa_index_select against the oracle")


@pytest.mark.parametrize("kind", ["index_select", "dense_prefill", "dense_decode"])
def test_graph_replays_equal_eager(kind):
    """The calls allocate nothing and clear nothing with memsets, so they can be
    captured in a HIP graph: every replay (with eager work in between) must
    equal the eager call."""
    decode = kind == "dense_decode"
    w = (M2.with_sizes("graph_dec", [3000 + 113 * i for i in range(6)], [1] * 6, permuted_table=True) if decode
         else M2.with_sizes("graph_pre", [5000], [2500]))
    _announce(f"graph {kind}: {w.seq_lens[:3]} {w.q_lens[:3]}")
    runner = MsaRunner(make_inputs(w, "cuda"))
    runner.step()
    inp = runner.inputs
    if kind == "index_select":
        # row-range chunks of 300 rows: the descriptor kernel runs before each chunk
        ws = torch.empty(256 + 300 * w.num_kv_heads * runner.ld * 4, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(runner.sel)
        call = lambda: ops.msa_index_select(runner.dims, runner.cache, runner.batch, inp.q_idx, out, ws)
    elif kind == "dense_prefill":
        out = torch.empty_like(inp.q)
        call = lambda: ops.msa_dense_attn_prefill(runner.dims, runner.cache, runner.batch, inp.q, out)
    else:
        need = ops.msa_workspace_size(runner.dims, runner.cache, runner.batch, ops.MSA_CALL_DENSE_ATTN_DECODE)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(inp.q)
        call = lambda: ops.msa_dense_attn_decode(runner.dims, runner.cache, runner.batch, inp.q, out, ws)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(4):
        out.fill_(-1 if out.dtype == torch.int32 else float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
        runner.step()  # eager work between replays
        torch.cuda.synchronize()

"""Guard bands around every buffer a call writes (robustness tier).

Each output, the cache and the workspace live inside a larger allocation
whose head and tail are filled with a sentinel; after the calls the
sentinels must be intact, so no kernel writes past either end of what it
was given.  The results themselves must equal those of the same calls on
ordinary buffers.
"""
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import ops
from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs
from block_sparse_long_score_amd.pipeline import MsaRunner

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements on each side (a multiple of 16 bytes for every dtype used)
SENTINEL = {torch.bfloat16: -3.0, torch.float32: -7.25, torch.int32: 0x5A5A5A5A, torch.uint8: 0xA5}

M2 = WORKLOADS["c1"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


class Guarded:
    """A view of `shape` inside a sentinel-filled allocation."""

    def __init__(self, shape, dtype, like=None):
        n = int(np.prod(shape))
        self.fill = SENTINEL[dtype]
        self.full = torch.full((n + 2 * GUARD,), self.fill, dtype=dtype, device="cuda")
        self.view = self.full[GUARD:GUARD + n].view(shape)
        if like is not None:
            self.view.copy_(like)

    def intact(self) -> bool:
        return bool((self.full[:GUARD] == self.fill).all()) and bool((self.full[-GUARD:] == self.fill).all())


def _guard_runner(runner):
    """Move the runner's cache, outputs and workspace into guarded buffers."""
    c = runner.cache
    guards = {
        "k cache": Guarded(c.k.shape, torch.bfloat16, c.k),
        "v cache": Guarded(c.v.shape, torch.bfloat16, c.v),
        "k_idx cache": Guarded(c.k_idx.shape, torch.bfloat16, c.k_idx),
        "block scores": Guarded(runner.scores.shape, torch.float32),
        "selections": Guarded(runner.sel.shape, torch.int32),
        "output": Guarded(runner.out.shape, torch.bfloat16),
        "workspace": Guarded(runner.workspace.shape, torch.uint8),
    }
    runner.cache = ops.Cache(guards["k cache"].view, guards["v cache"].view, guards["k_idx cache"].view,
                             c.block_table)
    runner.scores = guards["block scores"].view
    runner.sel = guards["selections"].view
    runner.out = guards["output"].view
    runner.workspace = guards["workspace"].view
    return guards


CASES = {
    "ragged_prefill": M2.with_sizes("g_ragged", [3001], [3001]),
    "chunk_mid_block": M2.with_sizes("g_chunk", [5000], [777]),
    "multi_seq": M2.with_sizes("g_multi", [2500, 129, 1, 4100], [2500, 60, 1, 900], permuted_table=True),
    "decode_fused": M2.with_sizes("g_dec_fused", [3000 + 97 * i for i in range(16)], [1] * 16, permuted_table=True),
    "decode_split": M2.with_sizes("g_dec_split", [1, 129, 2049, 9999], [1] * 4, permuted_table=True),
    "tiny_d64": WORKLOADS["c0"].with_sizes("g_c0", [2600], [2600]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_no_write_outside_any_buffer(name):
    w = CASES[name]
    _announce(f"guards {name}: seq_lens={w.seq_lens} q_lens={w.q_lens}")
    inputs = make_inputs(w, "cuda")
    ref = MsaRunner(inputs)
    ref.step()
    runner = MsaRunner(inputs)
    guards = _guard_runner(runner)
    runner.step()
    torch.cuda.synchronize()
    for what, g in guards.items():
        assert g.intact(), f"{name}: write outside the {what}"
    assert torch.equal(runner.sel, ref.sel)
    assert torch.equal(runner.out, ref.out)

    # the dense calls and the selection-quality calls, on guarded outputs
    dense = Guarded(runner.out.shape, torch.bfloat16)
    if runner.decode:
        need = ops.msa_workspace_size(runner.dims, runner.cache, runner.batch, ops.MSA_CALL_DENSE_ATTN_DECODE)
        ws = Guarded((need,), torch.uint8)
        ops.msa_dense_attn_decode(runner.dims, runner.cache, runner.batch, inputs.q, dense.view, ws.view)
        extra = {"dense output": dense, "dense workspace": ws}
    else:
        ops.msa_dense_attn_prefill(runner.dims, runner.cache, runner.batch, inputs.q, dense.view)
        extra = {"dense output": dense}
    rows = torch.from_numpy(np.unique(np.linspace(0, w.total_q - 1, 8).astype(np.int32))).cuda()
    mass = Guarded((rows.numel(), w.num_kv_heads, runner.ld), torch.float32)
    sel_mass = Guarded((rows.numel(), w.num_kv_heads, runner.ld), torch.float32)
    quality = Guarded((rows.numel(), w.num_kv_heads, 3), torch.float32)
    ops.msa_block_attn_mass(runner.dims, runner.cache, runner.batch, inputs.q, rows, mass.view)
    ops.msa_block_attn_mass(runner.dims, runner.cache, runner.batch, inputs.q, rows, sel_mass.view, sel=runner.sel)
    ops.msa_selection_quality(runner.dims, runner.batch, rows, mass.view, sel_mass.view, runner.scores, runner.sel,
                              quality.view)
    torch.cuda.synchronize()
    extra.update({"attention mass": mass, "candidate mass": sel_mass, "quality": quality})
    for what, g in {**guards, **extra}.items():
        assert g.intact(), f"{name}: write outside the {what}"

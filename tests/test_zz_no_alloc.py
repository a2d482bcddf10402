"""msa_sparse_attn_decode_noalloc (the decode Main Branch on the library's
static scratch, for callers that cannot allocate) against
msa_sparse_attn_decode with a caller workspace: identical outputs, bit for
bit, on two calls in a row (the second on a smaller batch, so it runs over
what the first left in the scratch), for the split decode (fewer than 128
(sequence, group) pairs, which uses the scratch for partial rows), the
two-workgroups-per-pair decode (128 to 255 pairs, which keeps the halves'
state and the pair counters there) and the one-workgroup-per-pair decode
(256 pairs or more, which needs none), including a batch near the scratch's
capacity."""
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import ops
from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs
from block_sparse_long_score_amd.pipeline import MsaRunner
from tests.gpu_helpers import compare_rows

pytestmark = pytest.mark.gpu

M2 = WORKLOADS["c1"]
_LENS = [1, 128, 129, 2047, 2049, 5000, 16 * 128, 16 * 128 + 1, 300, 4097, 7777, 12000, 64, 1500, 2176, 9000]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(name):
    if name == "split_then_smaller":
        return [M2.with_sizes("na_split7", _LENS[:7], [1] * 7, permuted_table=True),
                M2.with_sizes("na_split3", _LENS[7:10], [1] * 3, permuted_table=True)]
    if name == "fused_then_split":
        return [M2.with_sizes("na_fused16", _LENS, [1] * 16, permuted_table=True),
                M2.with_sizes("na_split2", [9999, 3000], [1, 1], permuted_table=True)]
    if name == "whole_then_half":  # 256 pairs, then 192
        return [M2.with_sizes("na_whole32", [_LENS[i % 16] + 3 * i for i in range(32)], [1] * 32, permuted_table=True),
                M2.with_sizes("na_half24", [_LENS[i % 16] + 5 * i for i in range(24)], [1] * 24, permuted_table=True)]
    if name == "half_then_half":  # 192 pairs, then 128 (the counters of the first must not leak into the second)
        return [M2.with_sizes("na_half24b", [_LENS[i % 16] + 7 * i for i in range(24)], [1] * 24, permuted_table=True),
                M2.with_sizes("na_half16", _LENS, [1] * 16, permuted_table=True)]
    # M3 shape (G = 16): 31 sequences x 4 groups = 124 pairs, close to the scratch's capacity
    m3 = WORKLOADS["m3d"]
    lens = [_LENS[i % 16] + 11 * i for i in range(31)]
    return [m3.with_sizes("na_m3_31", lens, [1] * 31, permuted_table=True),
            m3.with_sizes("na_m3_5", lens[:5], [1] * 5, permuted_table=True)]


@pytest.mark.parametrize("name", ["split_then_smaller", "fused_then_split", "whole_then_half", "half_then_half",
                                  "near_capacity"])
def test_noalloc_decode_equals_workspace_decode(name):
    for i, w in enumerate(_case(name)):
        print(f"[gpu-case] {name} call {i}: {w.name} num_seqs={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads}",
              flush=True)
        sys.stdout.flush()
        runner = MsaRunner(make_inputs(w, "cuda"))
        runner.step()  # the workspace decode: runner.out
        torch.cuda.synchronize()
        got = torch.full_like(runner.out, float("nan"))
        ops.msa_sparse_attn_decode_noalloc(runner.dims, runner.cache, runner.batch, runner.inputs.q, runner.sel, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), runner.out.view(torch.int16)), f"{w.name}: outputs differ"
        for s in range(w.num_seqs):  # and the oracle, on every row
            compare_rows(runner, s, [w.seq_lens[s] - 1], check_scores=False)
        need = ops.msa_workspace_size(runner.dims, runner.cache, runner.batch, ops.MSA_CALL_SPARSE_ATTN_DECODE)
        pairs = w.num_seqs * w.num_kv_heads
        if pairs < 128:
            assert need <= 8_583_168, need

"""One MSA step over a synthetic workload, through the C ABI.

A step is the whole hot path for one batch: append the new tokens' K, V and
K_idx to the block-major cache, score and max-pool the index branch, select
the blocks, and run the Main Branch (prefill or decode).  The runner holds the
device buffers; it does no arithmetic of its own.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops
from .inputs import Inputs


class MsaRunner:
    def __init__(self, inputs: Inputs):
        w = inputs.workload
        dev = inputs.q.device
        self.inputs = inputs
        self.dims = ops.Dims(w.num_q_heads, w.num_kv_heads, w.head_dim, w.index_dim, w.block_size, w.top_k)
        self.cache = ops.Cache.allocate(self.dims, inputs.num_blocks, inputs.block_table)
        self.batch = ops.Batch.make(w.seq_lens, w.q_lens, dev)
        self.decode = all(n == 1 for n in w.q_lens)
        self._fill_prefix()
        rows = inputs.new_token_rows()
        self.k_new = inputs.k.index_select(0, rows).contiguous()
        self.v_new = inputs.v.index_select(0, rows).contiguous()
        self.k_idx_new = inputs.k_idx.index_select(0, rows).contiguous()
        self.ld = self.batch.max_blocks
        self.scores = torch.empty((w.total_q, w.num_kv_heads, self.ld), dtype=torch.float32, device=dev)
        self.sel = torch.empty((w.total_q, w.num_kv_heads, w.top_k), dtype=torch.int32, device=dev)
        self.out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        call = ops.MSA_CALL_SPARSE_ATTN_DECODE if self.decode else ops.MSA_CALL_SPARSE_ATTN_PREFILL
        self.workspace = torch.empty(ops.msa_workspace_size(self.dims, self.cache, self.batch, call),
                                     dtype=torch.uint8, device=dev)

    def _fill_prefix(self):
        """Cache every token before the step's queries, one sequence at a time."""
        w, inp = self.inputs.workload, self.inputs
        off = inp.tok_off
        prefix = np.array([n - nq for n, nq in zip(w.seq_lens, w.q_lens)], dtype=np.int64)
        for s in range(w.num_seqs):
            if prefix[s] == 0:
                continue
            q_lens = np.zeros(w.num_seqs, dtype=np.int64)
            q_lens[s] = prefix[s]
            b = ops.Batch.make(prefix, q_lens, inp.q.device)
            lo, hi = int(off[s]), int(off[s] + prefix[s])
            ops.msa_kv_append(self.dims, self.cache, b, inp.k[lo:hi], inp.v[lo:hi], inp.k_idx[lo:hi])

    # The four calls of one step, exposed separately so they can be timed.
    def append(self, stream=None):
        ops.msa_kv_append(self.dims, self.cache, self.batch, self.k_new, self.v_new, self.k_idx_new, stream)

    def index_score(self, stream=None):
        ops.msa_index_score(self.dims, self.cache, self.batch, self.inputs.q_idx, self.scores, stream)

    def block_topk(self, stream=None):
        ops.msa_block_topk(self.dims, self.batch, self.scores, self.sel, stream)

    def attend(self, sel=None, stream=None):
        sel = self.sel if sel is None else sel
        fn = ops.msa_sparse_attn_decode if self.decode else ops.msa_sparse_attn_prefill
        fn(self.dims, self.cache, self.batch, self.inputs.q, sel, self.out, self.workspace, stream)

    def step(self, stream=None):
        self.append(stream)
        self.index_score(stream)
        self.block_topk(stream)
        self.attend(stream=stream)

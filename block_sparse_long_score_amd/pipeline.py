"""One MSA step over a synthetic workload, through the C ABI.

A step is the whole hot path for one batch: append the new tokens' K, V and
K_idx to the block-major cache, score and max-pool the index branch, select
the blocks, and run the Main Branch (prefill or decode).  The runner holds the
device buffers; it does no arithmetic of its own.

Pipelined prefill.  The index branch is bound by the matrix cores and the
Main Branch by HBM bandwidth, so a long prefill is cut into chunks of query
rows (each chunk is an ordinary prefill chunk: its queries are the last rows
of a sequence truncated after the chunk).  Scoring and selection of chunk i+1
run on the caller's stream while the Main Branch of chunk i runs on a second
stream of the same (default) priority; events order each chunk's attention
after its own selection, and the caller's stream waits for the last one.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops
from .inputs import Inputs


class MsaRunner:
    """fused_decode (decode batches; default on): a step is one msa_decode_step
    call (append, scoring, selection and attention in two kernels) instead of
    the four separate calls; results are the same bit for bit."""

    def __init__(self, inputs: Inputs, chunk_rows: int | None = None, fused_decode: bool = True):
        w = inputs.workload
        dev = inputs.q.device
        self.inputs = inputs
        self.dims = ops.Dims(w.num_q_heads, w.num_kv_heads, w.head_dim, w.index_dim, w.block_size, w.top_k)
        self.cache = ops.Cache.allocate(self.dims, inputs.num_blocks, inputs.block_table)
        self.batch = ops.Batch.make(w.seq_lens, w.q_lens, dev)
        self.decode = all(n == 1 for n in w.q_lens)
        self.fused_decode = self.decode and fused_decode
        self._fill_prefix()
        rows = inputs.new_token_rows()
        self.k_new = inputs.k.index_select(0, rows).contiguous()
        self.v_new = inputs.v.index_select(0, rows).contiguous()
        self.k_idx_new = inputs.k_idx.index_select(0, rows).contiguous()
        self.ld = self.batch.max_blocks
        self.scores = torch.empty((w.total_q, w.num_kv_heads, self.ld), dtype=torch.float32, device=dev)
        self.sel = torch.empty((w.total_q, w.num_kv_heads, w.top_k), dtype=torch.int32, device=dev)
        self.out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        self.chunks = []
        if chunk_rows and not self.decode and w.num_seqs == 1 and w.q_lens[0] > chunk_rows:
            first = w.seq_lens[0] - w.q_lens[0]
            for r0 in range(0, w.q_lens[0], chunk_rows):
                r1 = min(r0 + chunk_rows, w.q_lens[0])
                self.chunks.append((r0, r1, ops.Batch.make([first + r1], [r1 - r0], dev)))
            self.stream_b = torch.cuda.Stream(device=dev)  # default priority
            self.events = [torch.cuda.Event() for _ in range(len(self.chunks) + 1)]
        ws_batch = self.chunks[0][2] if self.chunks else self.batch
        calls = ([ops.MSA_CALL_SPARSE_ATTN_DECODE, ops.MSA_CALL_DECODE_STEP] if self.decode
                 else [ops.MSA_CALL_SPARSE_ATTN_PREFILL])
        self.workspace = torch.empty(max(ops.msa_workspace_size(self.dims, self.cache, ws_batch, c) for c in calls),
                                     dtype=torch.uint8, device=dev)
        # Optional observer: hook(stage, stream, phase) is called right before
        # (phase 0) and after (phase 1) each stage is enqueued in step(), with
        # the stream it is enqueued on (used to time a stage with events).
        self.hook = None
        self._prepared, self._prepared_key = None, None

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

    def _calls(self):
        """The step's C-ABI calls with their arguments marshalled once
        (ops.prepare), so a step's host work stays far below its GPU time.
        Rebuilt whenever one of the runner's buffers has been replaced: the
        key is the identity of each object the calls were prepared from.
        Cache and Batch are frozen, so their tensors cannot be swapped behind
        an unchanged wrapper, and each prepared call keeps the buffers it
        captured alive, so no identity is reused while it exists."""
        inp = self.inputs
        key = tuple(map(id, (self.cache, self.batch, self.scores, self.sel, self.out, self.workspace, self.k_new,
                             self.v_new, self.k_idx_new, inp.q, inp.q_idx)))
        if key != self._prepared_key:
            attn = "msa_sparse_attn_decode" if self.decode else "msa_sparse_attn_prefill"
            whole = {
                "append": ops.prepare("msa_kv_append", self.dims, self.cache, self.batch, self.k_new, self.v_new,
                                      self.k_idx_new),
                "index_score": ops.prepare("msa_index_score", self.dims, self.cache, self.batch, inp.q_idx,
                                           self.scores),
                "block_topk": ops.prepare("msa_block_topk", self.dims, self.batch, self.scores, self.sel),
                "attend": ops.prepare(attn, self.dims, self.cache, self.batch, inp.q, self.sel, self.out,
                                      self.workspace),
            }
            if self.decode:
                whole["decode_step"] = ops.prepare("msa_decode_step", self.dims, self.cache, self.batch, self.k_new,
                                                   self.v_new, self.k_idx_new, inp.q_idx, inp.q, self.scores,
                                                   self.sel, self.out, self.workspace)
            chunks = []
            for r0, r1, cb in self.chunks:
                scores, sel = self.scores[r0:r1], self.sel[r0:r1]
                chunks.append({
                    "index_score": ops.prepare("msa_index_score", self.dims, self.cache, cb, inp.q_idx[r0:r1], scores),
                    "block_topk": ops.prepare("msa_block_topk", self.dims, cb, scores, sel),
                    "attend": ops.prepare("msa_sparse_attn_prefill", self.dims, self.cache, cb, inp.q[r0:r1], sel,
                                          self.out[r0:r1], self.workspace),
                })
            self._prepared, self._prepared_key = (whole, chunks), key
        return self._prepared

    # The four calls of one step, exposed separately so they can be timed.
    def append(self, stream=None):
        self._calls()[0]["append"](stream)

    def index_score(self, stream=None):
        self._calls()[0]["index_score"](stream)

    def block_topk(self, stream=None):
        self._calls()[0]["block_topk"](stream)

    def attend(self, sel=None, stream=None):
        if sel is not None and sel is not self.sel:
            fn = ops.msa_sparse_attn_decode if self.decode else ops.msa_sparse_attn_prefill
            return fn(self.dims, self.cache, self.batch, self.inputs.q, sel, self.out, self.workspace, stream)
        self._calls()[0]["attend"](stream)

    def _stage(self, name, stream, fn):
        if self.hook is None:
            return fn()
        self.hook(name, stream, 0)
        fn()
        self.hook(name, stream, 1)

    def step(self, stream=None, fused: bool | None = None):
        """One step.  fused (decode only; default: the runner's fused_decode):
        one msa_decode_step call, else the four calls one by one (the hook, if
        set, then sees each of them)."""
        if self.chunks:
            return self.pipelined_step()
        st = stream if stream is not None else torch.cuda.current_stream()
        calls = self._calls()[0]
        if self.decode and (self.fused_decode if fused is None else fused):
            return self._stage("decode_step", st, lambda: calls["decode_step"](st))
        if self.hook is None:
            for name in ("append", "index_score", "block_topk", "attend"):
                calls[name](st)
            return
        for name in ("append", "index_score", "block_topk", "attend"):
            self._stage(name, st, lambda: calls[name](st))

    def capture(self):
        """Record one unchunked step as a HIP graph, so that replay() issues
        the whole step with a single launch from the host.  The step's kernels
        allocate nothing and clear nothing with memset nodes; every buffer is
        the runner's own, so replays are the same work on the same memory."""
        if self.chunks:
            raise ValueError("a chunked (two-stream) prefill step is not captured")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.step()

    def replay(self):
        self.graph.replay()

    def staged_step(self, mark):
        """The step run serially on the current stream, calling mark(name)
        after each stage (chunk by chunk when chunked) so a caller can record
        an event there.  Used to time the stages one by one."""
        a = torch.cuda.current_stream()
        whole, chunks = self._calls()
        mark("start")
        whole["append"](a)
        mark("append")
        for calls in chunks or [whole]:
            calls["index_score"](a)
            mark("index_score")
            calls["block_topk"](a)
            mark("block_topk")
            calls["attend"](a)
            mark("attend")

    def pipelined_step(self):
        """The same step, chunked over query rows with scoring/selection and
        attention of consecutive chunks overlapped on two streams."""
        a = torch.cuda.current_stream()
        b = self.stream_b
        whole, chunks = self._calls()
        self._stage("append", a, lambda: whole["append"](a))
        for i, calls in enumerate(chunks):
            self._stage("index_score", a, lambda: calls["index_score"](a))
            self._stage("block_topk", a, lambda: calls["block_topk"](a))
            self.events[i].record(a)
            b.wait_event(self.events[i])
            self._stage("attend", b, lambda: calls["attend"](b))
        self.events[-1].record(b)
        a.wait_event(self.events[-1])

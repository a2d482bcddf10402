"""Python binding of libmsa with the C ABI's entry-point names.

Argument marshalling only: tensors become device pointers, host mirrors
become host pointers, and the call is enqueued on the current HIP stream (or
the one given).  Every step of the computation runs in the library's kernels;
a failing status raises MsaError with the library's own message.
"""
from __future__ import annotations

import ctypes
import dataclasses

import numpy as np
import torch

from . import _lib
from ._lib import (MSA_CALL_DECODE_STEP, MSA_CALL_DENSE_ATTN_DECODE, MSA_CALL_INDEX_SELECT, MSA_CALL_SPARSE_ATTN_DECODE,
                   MSA_CALL_SPARSE_ATTN_PREFILL, MSA_CALL_SPARSE_ATTN_PREFILL_PLAN, MSA_CALL_SPARSE_ATTN_PREFILL_RUN,
                   MsaBatch, MsaCache, MsaDims)

__all__ = ["Dims", "Cache", "Batch", "MsaError", "msa_kv_append", "msa_index_score", "msa_block_topk",
           "msa_sparse_attn_prefill", "msa_sparse_attn_prefill_plan", "msa_sparse_attn_prefill_run",
           "msa_sparse_attn_decode", "msa_sparse_attn_decode_noalloc", "msa_dense_attn_prefill", "msa_dense_attn_decode",
           "msa_index_select", "msa_decode_step", "msa_block_attn_mass", "msa_selection_quality", "msa_workspace_size", "msa_abi_version",
           "PreparedCall", "prepare",
           "MSA_CALL_SPARSE_ATTN_PREFILL", "MSA_CALL_SPARSE_ATTN_DECODE", "MSA_CALL_DENSE_ATTN_DECODE", "MSA_CALL_INDEX_SELECT",
           "MSA_CALL_SPARSE_ATTN_PREFILL_PLAN", "MSA_CALL_SPARSE_ATTN_PREFILL_RUN", "MSA_CALL_DECODE_STEP"]


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_lib.STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


@dataclasses.dataclass(frozen=True)
class Dims:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    index_dim: int
    block_size: int = 128
    top_k: int = 16
    softmax_scale: float = 0.0  # <= 0: 1/sqrt(head_dim)

    def c(self) -> MsaDims:
        return MsaDims(self.num_q_heads, self.num_kv_heads, self.head_dim, self.index_dim, self.block_size,
                       self.top_k, self.softmax_scale)


@dataclasses.dataclass(frozen=True)
class Cache:
    """Block-major cache: k, v bf16 [num_blocks, 128, Hkv, D]; k_idx bf16
    [num_blocks, 128, d_idx]; block_table int32 [num_seqs, max_blocks_per_seq]."""
    k: torch.Tensor
    v: torch.Tensor
    k_idx: torch.Tensor
    block_table: torch.Tensor

    @staticmethod
    def allocate(dims: Dims, num_blocks: int, block_table: torch.Tensor) -> "Cache":
        dev = block_table.device
        shape = (num_blocks, dims.block_size, dims.num_kv_heads, dims.head_dim)
        return Cache(torch.empty(shape, dtype=torch.bfloat16, device=dev),
                     torch.empty(shape, dtype=torch.bfloat16, device=dev),
                     torch.empty((num_blocks, dims.block_size, dims.index_dim), dtype=torch.bfloat16, device=dev),
                     block_table.to(torch.int32).contiguous())

    def c(self) -> MsaCache:
        return MsaCache(self.k.data_ptr(), self.v.data_ptr(), self.k_idx.data_ptr(), self.block_table.data_ptr(),
                        self.k.shape[0], self.block_table.shape[1])


@dataclasses.dataclass(frozen=True)
class Batch:
    """seq_lens: tokens per sequence after this step's append; the queries of
    sequence s are its last cu_q[s+1]-cu_q[s] positions."""
    seq_lens: torch.Tensor  # device int32 [num_seqs]
    cu_q: torch.Tensor      # device int32 [num_seqs + 1]
    seq_lens_host: np.ndarray
    cu_q_host: np.ndarray

    @staticmethod
    def make(seq_lens, q_lens, device) -> "Batch":
        sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
        cu = np.ascontiguousarray(np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))]).astype(np.int32))
        return Batch(torch.from_numpy(sl).to(device), torch.from_numpy(cu).to(device), sl, cu)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens_host.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_q_host[-1])

    @property
    def max_blocks(self) -> int:
        return int(max(((int(n) + 127) // 128 for n in self.seq_lens_host), default=0))

    def c(self) -> MsaBatch:
        return MsaBatch(self.num_seqs, self.total_q, self.seq_lens.data_ptr(), self.cu_q.data_ptr(),
                        self.seq_lens_host.ctypes.data, self.cu_q_host.ctypes.data)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor, name: str, dtype) -> int:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check(status: int):
    if status != _lib.MSA_OK:
        raise MsaError(status, _lib.load().msa_last_error().decode())


def msa_abi_version() -> int:
    return int(_lib.load().msa_abi_version())


# Argument marshalling of the calls a step repeats: each returns the C
# arguments before the stream.  ctypes.byref keeps its struct alive.
def _kv_append_args(dims, cache, batch, k_new, v_new, k_idx_new):
    return (ctypes.byref(dims.c()), ctypes.byref(cache.c()), ctypes.byref(batch.c()),
            _ptr(k_new, "k_new", torch.bfloat16), _ptr(v_new, "v_new", torch.bfloat16),
            _ptr(k_idx_new, "k_idx_new", torch.bfloat16))


def _index_score_args(dims, cache, batch, q_idx, block_scores):
    return (ctypes.byref(dims.c()), ctypes.byref(cache.c()), ctypes.byref(batch.c()),
            _ptr(q_idx, "q_idx", torch.bfloat16), _ptr(block_scores, "block_scores", torch.float32),
            block_scores.shape[-1])


def _block_topk_args(dims, batch, block_scores, sel):
    return (ctypes.byref(dims.c()), ctypes.byref(batch.c()), _ptr(block_scores, "block_scores", torch.float32),
            block_scores.shape[-1], _ptr(sel, "sel", torch.int32))


def _attn_args(dims, cache, batch, q, sel, out, workspace):
    return (ctypes.byref(dims.c()), ctypes.byref(cache.c()), ctypes.byref(batch.c()), _ptr(q, "q", torch.bfloat16),
            _ptr(sel, "sel", torch.int32), _ptr(out, "out", torch.bfloat16),
            _ptr(workspace, "workspace", torch.uint8), workspace.numel())


def _decode_step_args(dims, cache, batch, k_new, v_new, k_idx_new, q_idx, q, block_scores, sel, out, workspace):
    return (ctypes.byref(dims.c()), ctypes.byref(cache.c()), ctypes.byref(batch.c()),
            _ptr(k_new, "k_new", torch.bfloat16), _ptr(v_new, "v_new", torch.bfloat16),
            _ptr(k_idx_new, "k_idx_new", torch.bfloat16), _ptr(q_idx, "q_idx", torch.bfloat16),
            _ptr(q, "q", torch.bfloat16), _ptr(block_scores, "block_scores", torch.float32), block_scores.shape[-1],
            _ptr(sel, "sel", torch.int32), _ptr(out, "out", torch.bfloat16),
            _ptr(workspace, "workspace", torch.uint8), workspace.numel())


_MARSHAL = {"msa_kv_append": _kv_append_args, "msa_index_score": _index_score_args,
            "msa_block_topk": _block_topk_args, "msa_sparse_attn_prefill": _attn_args,
            "msa_sparse_attn_decode": _attn_args, "msa_decode_step": _decode_step_args}


def _buffers(obj):
    """The tensors and host arrays whose addresses a call's arguments carry."""
    if isinstance(obj, Cache):
        return [obj.k, obj.v, obj.k_idx, obj.block_table]
    if isinstance(obj, Batch):
        return [obj.seq_lens, obj.cu_q, obj.seq_lens_host, obj.cu_q_host]
    if isinstance(obj, (torch.Tensor, np.ndarray)):
        return [obj]
    return []


class PreparedCall:
    """One C-ABI call with its arguments marshalled once, for loops that repeat
    the same call on the same buffers (a decode or prefill step): calling it
    costs one ctypes call (the library still validates every argument)
    instead of rebuilding the structs and re-checking every tensor.  It keeps
    every tensor and host array whose address it captured alive (not only
    the Cache / Batch wrappers, whose fields could be reassigned), so the
    captured addresses stay valid for as long as the call exists; their
    contents may change between calls."""
    __slots__ = ("_fn", "_args", "_keep")

    def __init__(self, name, args, keep):
        self._fn = getattr(_lib.load(), name)
        self._args = args
        self._keep = keep

    def __call__(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)))


def prepare(name: str, *args) -> PreparedCall:
    """PreparedCall for one of msa_kv_append, msa_index_score, msa_block_topk,
    msa_sparse_attn_prefill, msa_sparse_attn_decode, msa_decode_step, with the
    same positional arguments as the function of that name (without the stream)."""
    keep = tuple(b for a in args for b in _buffers(a))
    return PreparedCall(name, _MARSHAL[name](*args), keep)


def msa_kv_append(dims: Dims, cache: Cache, batch: Batch, k_new, v_new, k_idx_new, stream=None):
    _check(_lib.load().msa_kv_append(*_kv_append_args(dims, cache, batch, k_new, v_new, k_idx_new), _stream(stream)))


def msa_index_score(dims: Dims, cache: Cache, batch: Batch, q_idx, block_scores, stream=None):
    """block_scores: float32 [total_q, Hkv, ld]; entries after each row's block are left untouched."""
    _check(_lib.load().msa_index_score(*_index_score_args(dims, cache, batch, q_idx, block_scores), _stream(stream)))


def msa_block_topk(dims: Dims, batch: Batch, block_scores, sel, stream=None):
    _check(_lib.load().msa_block_topk(*_block_topk_args(dims, batch, block_scores, sel), _stream(stream)))


def msa_workspace_size(dims: Dims, cache: Cache, batch: Batch, call: int) -> int:
    L = _lib.load()
    d, c, b = dims.c(), cache.c(), batch.c()
    n = int(L.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b), call))
    if n == 0:
        raise MsaError(2, L.msa_last_error().decode())
    return n


def _attn(fn_name, dims, cache, batch, q, sel, out, workspace, stream):
    _check(getattr(_lib.load(), fn_name)(*_attn_args(dims, cache, batch, q, sel, out, workspace), _stream(stream)))


def msa_sparse_attn_prefill(dims: Dims, cache: Cache, batch: Batch, q, sel, out, workspace, stream=None):
    _attn("msa_sparse_attn_prefill", dims, cache, batch, q, sel, out, workspace, stream)


def msa_sparse_attn_prefill_plan(dims: Dims, cache: Cache, batch: Batch, sel, plan, stream=None):
    """plan: uint8, at least msa_workspace_size(..., MSA_CALL_SPARSE_ATTN_PREFILL_PLAN) bytes."""
    L = _lib.load()
    d, c, b = dims.c(), cache.c(), batch.c()
    _check(L.msa_sparse_attn_prefill_plan(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b),
                                          _ptr(sel, "sel", torch.int32), _ptr(plan, "plan", torch.uint8),
                                          plan.numel(), _stream(stream)))


def msa_sparse_attn_prefill_run(dims: Dims, cache: Cache, batch: Batch, q, sel, plan, out, workspace, stream=None):
    """plan: as written by msa_sparse_attn_prefill_plan for the same dims, cache, batch and sel;
    workspace: uint8, at least msa_workspace_size(..., MSA_CALL_SPARSE_ATTN_PREFILL_RUN) bytes."""
    L = _lib.load()
    d, c, b = dims.c(), cache.c(), batch.c()
    _check(L.msa_sparse_attn_prefill_run(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b),
                                         _ptr(q, "q", torch.bfloat16), _ptr(sel, "sel", torch.int32),
                                         _ptr(plan, "plan", torch.uint8), _ptr(out, "out", torch.bfloat16),
                                         _ptr(workspace, "workspace", torch.uint8), workspace.numel(),
                                         _stream(stream)))


def msa_sparse_attn_decode(dims: Dims, cache: Cache, batch: Batch, q, sel, out, workspace, stream=None):
    _attn("msa_sparse_attn_decode", dims, cache, batch, q, sel, out, workspace, stream)


def msa_decode_step(dims: Dims, cache: Cache, batch: Batch, k_new, v_new, k_idx_new, q_idx, q, block_scores, sel, out,
                    workspace, stream=None):
    """One decode step (msa_kv_append, msa_index_score, msa_block_topk and msa_sparse_attn_decode in
    sequence, same results) as two kernels; workspace: uint8, at least
    msa_workspace_size(..., MSA_CALL_DECODE_STEP) bytes."""
    _check(_lib.load().msa_decode_step(*_decode_step_args(dims, cache, batch, k_new, v_new, k_idx_new, q_idx, q,
                                                          block_scores, sel, out, workspace), _stream(stream)))


def msa_sparse_attn_decode_noalloc(dims: Dims, cache: Cache, batch: Batch, q, sel, out, stream=None):
    """msa_sparse_attn_decode with the library's static scratch instead of a workspace
    (for callers that cannot allocate); calls that overlap on one GPU race."""
    L = _lib.load()
    d, c, b = dims.c(), cache.c(), batch.c()
    _check(L.msa_sparse_attn_decode_noalloc(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b),
                                            _ptr(q, "q", torch.bfloat16), _ptr(sel, "sel", torch.int32),
                                            _ptr(out, "out", torch.bfloat16), _stream(stream)))


def msa_index_select(dims: Dims, cache: Cache, batch: Batch, q_idx, sel, workspace, stream=None):
    """Scoring, pooling and top-k in one call, chunked through `workspace` (uint8; the chunk
    size follows its size); sel: int32 [total_q, Hkv, top_k], identical to the two calls'."""
    L = _lib.load()
    d, c, b = dims.c(), cache.c(), batch.c()
    _check(L.msa_index_select(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b), _ptr(q_idx, "q_idx", torch.bfloat16),
                              _ptr(sel, "sel", torch.int32), _ptr(workspace, "workspace", torch.uint8),
                              workspace.numel(), _stream(stream)))


def msa_dense_attn_prefill(dims: Dims, cache: Cache, batch: Batch, q, out, stream=None):
    """Dense causal attention of every query row over all its causal keys; out: bf16 [total_q, Hq, D]."""
    L = _lib.load()
    d, c, b = dims.c(), cache.c(), batch.c()
    _check(L.msa_dense_attn_prefill(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b), _ptr(q, "q", torch.bfloat16),
                                    _ptr(out, "out", torch.bfloat16), _stream(stream)))


def msa_dense_attn_decode(dims: Dims, cache: Cache, batch: Batch, q, out, workspace, stream=None):
    """Dense attention of one query row per sequence over its whole context; out: bf16 [num_seqs, Hq, D].
    workspace: uint8, at least msa_workspace_size(..., MSA_CALL_DENSE_ATTN_DECODE) bytes."""
    L = _lib.load()
    d, c, b = dims.c(), cache.c(), batch.c()
    _check(L.msa_dense_attn_decode(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b), _ptr(q, "q", torch.bfloat16),
                                   _ptr(out, "out", torch.bfloat16), _ptr(workspace, "workspace", torch.uint8),
                                   workspace.numel(), _stream(stream)))


def msa_block_attn_mass(dims: Dims, cache: Cache, batch: Batch, q, rows, mass, sel=None, stream=None):
    """mass: float32 [n_rows, Hkv, ld]; rows: int32 [n_rows] query-row indices of the batch.
    sel None: the dense mass over every causal token; sel (int32 [total_q, Hkv, top_k]): the
    Main Branch's mass over the tokens of the selected blocks."""
    L = _lib.load()
    d, c, b = dims.c(), cache.c(), batch.c()
    sel_ptr = None if sel is None else _ptr(sel, "sel", torch.int32)
    _check(L.msa_block_attn_mass(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b), _ptr(q, "q", torch.bfloat16),
                                 sel_ptr, _ptr(rows, "rows", torch.int32), rows.numel(),
                                 _ptr(mass, "mass", torch.float32), mass.shape[-1], _stream(stream)))


def msa_selection_quality(dims: Dims, batch: Batch, rows, mass, sel_mass, block_scores, sel, quality, stream=None):
    """quality: float32 [n_rows, Hkv, 3] = (coverage, recall, kl); mass is the dense mass,
    sel_mass the Main Branch's mass over the selected blocks (msa_block_attn_mass with sel)."""
    L = _lib.load()
    d, b = dims.c(), batch.c()
    if block_scores.shape[-1] != mass.shape[-1] or sel_mass.shape[-1] != mass.shape[-1]:
        raise ValueError("mass, sel_mass and block_scores must share the row pitch ld")
    _check(L.msa_selection_quality(ctypes.byref(d), ctypes.byref(b), _ptr(rows, "rows", torch.int32), rows.numel(),
                                   _ptr(mass, "mass", torch.float32), _ptr(sel_mass, "sel_mass", torch.float32),
                                   _ptr(block_scores, "block_scores", torch.float32), _ptr(sel, "sel", torch.int32),
                                   mass.shape[-1], _ptr(quality, "quality", torch.float32), _stream(stream)))

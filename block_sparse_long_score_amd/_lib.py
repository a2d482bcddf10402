"""ctypes loader for libmsa.so (the C ABI declared in include/msa.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

# MSA_LIBRARY names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the in-tree libmsa.so.
LIB_PATH = os.environ.get("MSA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK = 0
STATUS_NAMES = {0: "MSA_OK", 1: "MSA_ERR_NULL_POINTER", 2: "MSA_ERR_BAD_SHAPE", 3: "MSA_ERR_UNSUPPORTED",
                4: "MSA_ERR_MISALIGNED", 5: "MSA_ERR_CAPACITY", 6: "MSA_ERR_WORKSPACE", 7: "MSA_ERR_HIP"}
MSA_CALL_SPARSE_ATTN_PREFILL = 1
MSA_CALL_SPARSE_ATTN_DECODE = 2
MSA_CALL_DENSE_ATTN_DECODE = 3
MSA_CALL_INDEX_SELECT = 4
MSA_CALL_SPARSE_ATTN_PREFILL_PLAN = 5
MSA_CALL_SPARSE_ATTN_PREFILL_RUN = 6
MSA_CALL_DECODE_STEP = 7


class MsaDims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("index_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class MsaCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_idx", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32)]


class MsaBatch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_q", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
                ("cu_q", ctypes.c_void_p), ("seq_lens_host", ctypes.c_void_p), ("cu_q_host", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m block_sparse_long_score_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    dims, cache, batch = P(MsaDims), P(MsaCache), P(MsaBatch)
    sigs = {
        "msa_kv_append": ([dims, cache, batch, vp, vp, vp, vp], ctypes.c_int),
        "msa_index_score": ([dims, cache, batch, vp, vp, i64, vp], ctypes.c_int),
        "msa_block_topk": ([dims, batch, vp, i64, vp, vp], ctypes.c_int),
        "msa_sparse_attn_prefill": ([dims, cache, batch, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "msa_sparse_attn_decode": ([dims, cache, batch, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "msa_sparse_attn_decode_noalloc": ([dims, cache, batch, vp, vp, vp, vp], ctypes.c_int),
        "msa_decode_step": ([dims, cache, batch, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, sz, vp], ctypes.c_int),
        "msa_sparse_attn_prefill_plan": ([dims, cache, batch, vp, vp, sz, vp], ctypes.c_int),
        "msa_sparse_attn_prefill_run": ([dims, cache, batch, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "msa_block_attn_mass": ([dims, cache, batch, vp, vp, vp, i32, vp, i64, vp], ctypes.c_int),
        "msa_selection_quality": ([dims, batch, vp, i32, vp, vp, vp, vp, i64, vp, vp], ctypes.c_int),
        "msa_index_select": ([dims, cache, batch, vp, vp, vp, sz, vp], ctypes.c_int),
        "msa_dense_attn_prefill": ([dims, cache, batch, vp, vp, vp], ctypes.c_int),
        "msa_dense_attn_decode": ([dims, cache, batch, vp, vp, vp, sz, vp], ctypes.c_int),
        "msa_workspace_size": ([dims, cache, batch, i32], sz),
        "msa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "msa_last_error": ([], ctypes.c_char_p),
        "msa_abi_version": ([], ctypes.c_int32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib

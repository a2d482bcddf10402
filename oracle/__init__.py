"""CPU oracle of MiniMax Sparse Attention (MSA) — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU path
(``block_sparse_long_score_amd``) and never imports it.

The arithmetic lives in ``msa_oracle.c`` (plain C, double precision, one loop
per step of the method); this module only compiles it, loads it with ctypes
and marshals numpy arrays.  The steps follow "MiniMax 模型迭代与竞品分析：从
Text-01、M1、M2 到 M3", §2: index scoring against a shared K_idx, max-pooling
into 128-token blocks, top-16 selection with the local block forced in, and
exact softmax attention over the selected tokens.  The same section's
training and evaluation quantities are here too: the dense attention mass per
block with a selection's coverage of it and recall of its largest blocks,
and the indexer's training target, D_KL(P || Q) between the Main Branch's
group-averaged importance P over the candidate (selected) blocks and the
indexer's softmax Q over the same blocks.

All tensors are numpy arrays in plain logical order for ONE sequence:
bf16 inputs are passed as ``uint16`` bit patterns, keys are indexed by token
position, and query rows carry their absolute positions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmsa_oracle.so")
_lib = None

_ERRORS = {1: "bad argument", 2: "invalid selection", 3: "out of memory"}


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/libmsa_oracle.so`` with gcc + OpenMP."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.msa_oracle_block_scores.argtypes = [i64, p, p, i32, i32, p, i64, i32, p, i64]
        lib.msa_oracle_select.argtypes = [i64, p, p, i32, i64, i32, i32, p]
        lib.msa_oracle_attend.argtypes = [i64, p, p, i32, i32, i32, p, p, i64, p, i32, i32, dbl, p]
        lib.msa_oracle_block_mass.argtypes = [i64, p, p, i32, i32, i32, p, i64, i32, dbl, p, i64]
        lib.msa_oracle_selection_quality.argtypes = [i64, p, p, p, i32, i64, i32, i32, p, p]
        lib.msa_oracle_selected_mass.argtypes = [i64, p, p, i32, i32, i32, p, i64, p, i32, i32, dbl, p, i64]
        lib.msa_oracle_indexer_kl.argtypes = [i64, p, p, p, p, i32, i64, i32, i32, p]
        for f in (lib.msa_oracle_block_scores, lib.msa_oracle_select, lib.msa_oracle_attend,
                  lib.msa_oracle_block_mass, lib.msa_oracle_selection_quality, lib.msa_oracle_selected_mass,
                  lib.msa_oracle_indexer_kl):
            f.restype = ctypes.c_int
        lib.msa_oracle_num_threads.restype = ctypes.c_int
        lib.msa_oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.msa_oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def set_num_threads(n: int) -> None:
    """Threads for the oracle's OpenMP loops from now on."""
    _load().msa_oracle_set_num_threads(int(n))


def num_threads() -> int:
    """Host threads the oracle's OpenMP loops use."""
    return int(_load().msa_oracle_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def block_scores(pos, q_idx, k_idx, block_size: int = 128, ld: int | None = None) -> np.ndarray:
    """Steps 1-2: pooled index scores.

    pos   : int64 [n]            absolute positions of the query rows
    q_idx : uint16 [n, G, d_idx] bf16 bits, one index query per GQA group
    k_idx : uint16 [L, d_idx]    bf16 bits, one index key per token (shared)
    returns float32 [n, G, ld]; entries of blocks after the row's own block are -inf.
    """
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    q_idx, k_idx = _u16(q_idx), _u16(k_idx)
    n, groups, d_idx = q_idx.shape
    if ld is None:
        ld = int(pos.max()) // block_size + 1 if n else 1
    out = np.empty((n, groups, ld), dtype=np.float32)
    rc = _load().msa_oracle_block_scores(n, _ptr(pos), _ptr(q_idx), groups, d_idx, _ptr(k_idx),
                                         k_idx.shape[0], block_size, _ptr(out), ld)
    _check(rc, "block_scores")
    return out


def select(pos, pooled, block_size: int = 128, top_k: int = 16) -> np.ndarray:
    """Step 3: int32 [n, G, top_k] ascending block ids, -1 padded."""
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    pooled = np.ascontiguousarray(pooled, dtype=np.float32)
    n, groups, ld = pooled.shape
    out = np.empty((n, groups, top_k), dtype=np.int32)
    rc = _load().msa_oracle_select(n, _ptr(pos), _ptr(pooled), groups, ld, block_size, top_k, _ptr(out))
    _check(rc, "select")
    return out


def attend(pos, q, k, v, sel, block_size: int = 128, scale: float | None = None) -> np.ndarray:
    """Step 4: float64 [n, Hq, D] softmax attention over the selected tokens.

    q    : uint16 [n, Hq, D]; k, v : uint16 [L, G, D]; sel : int32 [n, G, top_k]
    scale defaults to 1/sqrt(D).
    """
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    q, k, v = _u16(q), _u16(k), _u16(v)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, hq, d = q.shape
    groups = k.shape[1]
    top_k = sel.shape[2]
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    out = np.empty((n, hq, d), dtype=np.float64)
    rc = _load().msa_oracle_attend(n, _ptr(pos), _ptr(q), hq, groups, d, _ptr(k), _ptr(v), k.shape[0],
                                   _ptr(sel), block_size, top_k, float(scale), _ptr(out))
    _check(rc, "attend")
    return out


def dense_attend(pos, q, k, v, block_size: int = 128, scale: float | None = None) -> np.ndarray:
    """Dense causal attention: float64 [n, Hq, D], every key i <= t attended.

    It is step 4 with every causal block selected (the full-attention layers
    beside MSA in "MiniMax 模型迭代与竞品分析" §2-§3).
    """
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    n = pos.shape[0]
    groups = np.asarray(k).shape[1]
    nblk = int(pos.max()) // block_size + 1 if n else 1
    sel = np.full((n, groups, nblk), -1, dtype=np.int32)
    for r in range(n):
        c = int(pos[r]) // block_size
        sel[r, :, : c + 1] = np.arange(c + 1, dtype=np.int32)
    return attend(pos, q, k, v, sel, block_size, scale)


def msa(pos, q_idx, k_idx, q, k, v, block_size: int = 128, top_k: int = 16, scale: float | None = None,
        ld: int | None = None):
    """All four steps for query rows of one sequence: (pooled, sel, out)."""
    pooled = block_scores(pos, q_idx, k_idx, block_size, ld)
    sel = select(pos, pooled, block_size, top_k)
    out = attend(pos, q, k, v, sel, block_size, scale)
    return pooled, sel, out


def block_mass(pos, q, k, block_size: int = 128, scale: float | None = None, ld: int | None = None) -> np.ndarray:
    """Step 5: float64 [n, G, ld] dense attention mass per block, averaged over
    each group's heads (0 for blocks after the row's own block).

    q : uint16 [n, Hq, D]; k : uint16 [L, G, D].  scale defaults to 1/sqrt(D).
    """
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    q, k = _u16(q), _u16(k)
    n, hq, d = q.shape
    groups = k.shape[1]
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if ld is None:
        ld = int(pos.max()) // block_size + 1 if n else 1
    out = np.empty((n, groups, ld), dtype=np.float64)
    rc = _load().msa_oracle_block_mass(n, _ptr(pos), _ptr(q), hq, groups, d, _ptr(k), k.shape[0], block_size,
                                       float(scale), _ptr(out), ld)
    _check(rc, "block_mass")
    return out


def selection_quality(pos, mass, sel, block_size: int = 128):
    """Step 6: (coverage, recall), each float64 [n, G], of the selections
    against the dense mass.

    mass : float64 [n, G, ld] (converted if given as float32); sel : int32 [n, G, top_k].
    """
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    mass = np.ascontiguousarray(mass, dtype=np.float64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, groups, ld = mass.shape
    top_k = sel.shape[2]
    cov, rec = (np.empty((n, groups), dtype=np.float64) for _ in range(2))
    rc = _load().msa_oracle_selection_quality(n, _ptr(pos), _ptr(mass), _ptr(sel), groups, ld, block_size, top_k,
                                              _ptr(cov), _ptr(rec))
    _check(rc, "selection_quality")
    return cov, rec


def selected_mass(pos, q, k, sel, block_size: int = 128, scale: float | None = None,
                  ld: int | None = None) -> np.ndarray:
    """Step 7: float64 [n, G, ld], the Main Branch's group-averaged softmax mass
    of each selected block (its softmax runs over the selected tokens only);
    0 for every block that is not selected.

    q : uint16 [n, Hq, D]; k : uint16 [L, G, D]; sel : int32 [n, G, top_k].
    """
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    q, k = _u16(q), _u16(k)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, hq, d = q.shape
    groups = k.shape[1]
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if ld is None:
        ld = int(pos.max()) // block_size + 1 if n else 1
    out = np.empty((n, groups, ld), dtype=np.float64)
    rc = _load().msa_oracle_selected_mass(n, _ptr(pos), _ptr(q), hq, groups, d, _ptr(k), k.shape[0], _ptr(sel),
                                          block_size, sel.shape[2], float(scale), _ptr(out), ld)
    _check(rc, "selected_mass")
    return out


def indexer_kl(pos, sel_mass, pooled, sel, block_size: int = 128) -> np.ndarray:
    """Step 8: float64 [n, G], D_KL(P || Q) over each row's selected blocks,
    P = sel_mass (step 7), Q = softmax of the pooled index scores over the
    same blocks.

    sel_mass : float64 [n, G, ld]; pooled : float32 [n, G, ld]; sel : int32 [n, G, top_k].
    """
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel_mass = np.ascontiguousarray(sel_mass, dtype=np.float64)
    pooled = np.ascontiguousarray(pooled, dtype=np.float32)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n, groups, ld = sel_mass.shape
    if pooled.shape != sel_mass.shape:
        raise ValueError("sel_mass and pooled scores must have the same shape")
    kl = np.empty((n, groups), dtype=np.float64)
    rc = _load().msa_oracle_indexer_kl(n, _ptr(pos), _ptr(sel_mass), _ptr(pooled), _ptr(sel), groups, ld,
                                       block_size, sel.shape[2], _ptr(kl))
    _check(rc, "indexer_kl")
    return kl

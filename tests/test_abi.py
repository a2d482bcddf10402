"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/msa.h, and rejects invalid arguments on the host
(before any HIP call) with the documented status codes."""
import ctypes
import os
import re

import numpy as np
import pytest

from block_sparse_long_score_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

OK, NULLP, SHAPE, UNSUP, MISAL, CAP, WS, HIP = range(8)
FAKE = 1 << 20  # a 16-byte aligned non-null address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_long_score_amd import build
        build.build()
    return _lib.load()


def _dims(**kw):
    base = dict(num_q_heads=48, num_kv_heads=8, head_dim=128, index_dim=64, block_size=128, top_k=16,
                softmax_scale=0.0)
    base.update(kw)
    return _lib.MsaDims(**base)


class _Batch:
    def __init__(self, seq_lens, q_lens):
        self.sl = np.asarray(seq_lens, np.int32)
        self.cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        self.c = _lib.MsaBatch(len(seq_lens), int(self.cu[-1]), FAKE, FAKE, self.sl.ctypes.data, self.cu.ctypes.data)


def _cache(num_blocks=64, mbps=16, **kw):
    base = dict(k=FAKE, v=FAKE, k_idx=FAKE, block_table=FAKE, num_blocks=num_blocks, max_blocks_per_seq=mbps)
    base.update(kw)
    return _lib.MsaCache(**base)


def test_exports_every_declared_entry_point(lib):
    decls = set(re.findall(r"^\S.*?\b(msa_\w+)\(", open(HEADER).read(), re.M))
    assert {"msa_kv_append", "msa_index_score", "msa_block_topk", "msa_sparse_attn_prefill",
            "msa_sparse_attn_decode"} <= decls
    for name in decls:
        assert hasattr(lib, name), f"{name} declared in msa.h but not exported"


def test_abi_version_matches_header(lib):
    m = re.search(r"#define MSA_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.msa_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.msa_status_string(code).decode() == name
    assert lib.msa_status_string(99).decode() == "MSA_ERR_UNKNOWN"


def _index(lib, dims, cache, batch, q_idx=FAKE, out=FAKE, ld=16):
    return lib.msa_index_score(ctypes.byref(dims), ctypes.byref(cache), ctypes.byref(batch.c), q_idx, out, ld, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), UNSUP), (dict(index_dim=48), UNSUP), (dict(block_size=64), UNSUP), (dict(top_k=8), UNSUP),
    (dict(num_kv_heads=6, num_q_heads=48), UNSUP), (dict(num_q_heads=44), SHAPE), (dict(num_q_heads=0), SHAPE),
    (dict(num_q_heads=8 * 32, num_kv_heads=8), UNSUP), (dict(softmax_scale=float("inf")), SHAPE),
])
def test_bad_dims(lib, kw, status):
    b = _Batch([1024], [1024])
    assert _index(lib, _dims(**kw), _cache(), b) == status
    assert lib.msa_last_error().decode() != ""


def test_bad_batch(lib):
    d, c = _dims(), _cache()
    assert _index(lib, d, c, _Batch([100], [101])) == SHAPE           # more queries than tokens
    assert _index(lib, d, c, _Batch([16 * 128 + 1], [1])) == CAP       # beyond max_blocks_per_seq
    b = _Batch([100, 100], [10, 10])
    b.cu[2] = 5
    assert _index(lib, d, c, b) == SHAPE                               # cu_q decreasing
    b = _Batch([100], [10])
    b.c.total_q = 11
    assert _index(lib, d, c, b) == SHAPE                               # total_q mismatch
    assert _index(lib, d, c, _Batch([2048], [2048]), ld=15) == SHAPE   # ld too small
    b = _Batch([100], [10])
    b.c.seq_lens_host = None
    assert _index(lib, d, c, b) == NULLP


def test_null_and_misaligned_pointers(lib):
    d, b = _dims(), _Batch([1024], [1024])
    assert _index(lib, d, _cache(k=None), b) == NULLP
    assert _index(lib, d, _cache(k_idx=FAKE + 8), b) == MISAL
    assert _index(lib, d, _cache(), b, q_idx=None) == NULLP
    assert _index(lib, d, _cache(), b, out=FAKE + 4) == MISAL
    assert lib.msa_index_score(None, ctypes.byref(_cache()), ctypes.byref(b.c), FAKE, FAKE, 16, None) == NULLP


def test_topk_and_append_validation(lib):
    d, b = _dims(), _Batch([1024], [1024])
    assert lib.msa_block_topk(ctypes.byref(d), ctypes.byref(b.c), FAKE, 4, FAKE, None) == SHAPE  # ld < 8 blocks
    assert lib.msa_block_topk(ctypes.byref(d), ctypes.byref(b.c), FAKE, 8, None, None) == NULLP
    c = _cache()
    assert lib.msa_kv_append(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c), FAKE, None, FAKE, None) == NULLP
    assert lib.msa_kv_append(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c), FAKE, FAKE, FAKE + 2, None) == MISAL


def test_attention_validation(lib):
    d, c = _dims(), _cache()
    b = _Batch([1024, 900], [1, 2])
    need = lib.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c), 2)
    assert need > 0
    args = (ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c), FAKE, FAKE, FAKE)
    assert lib.msa_sparse_attn_decode(*args, FAKE, need, None) == SHAPE  # sequence 1 has two queries
    b1 = _Batch([1024, 900], [1, 1])
    need1 = lib.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b1.c), 2)
    args1 = (ctypes.byref(d), ctypes.byref(c), ctypes.byref(b1.c), FAKE, FAKE, FAKE)
    assert lib.msa_sparse_attn_decode(*args1, FAKE, need1 - 1, None) == WS
    assert lib.msa_sparse_attn_decode(*args1, None, need1, None) == WS
    needp = lib.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c), 1)
    assert lib.msa_sparse_attn_prefill(*args, FAKE, needp - 1, None) == WS
    assert lib.msa_sparse_attn_prefill(*args, FAKE + 8, needp, None) == MISAL
    assert lib.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c), 99) == 0


def test_noalloc_decode_validates_on_the_host(lib):
    """The allocation-free decode rejects what msa_sparse_attn_decode rejects, before any HIP call."""
    d, c = _dims(), _cache()
    b = _Batch([1024, 900], [1, 2])
    args = (ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c))
    assert lib.msa_sparse_attn_decode_noalloc(*args, FAKE, FAKE, FAKE, None) == SHAPE  # two queries in sequence 1
    b1 = _Batch([1024, 900], [1, 1])
    args1 = (ctypes.byref(d), ctypes.byref(c), ctypes.byref(b1.c))
    assert lib.msa_sparse_attn_decode_noalloc(*args1, None, FAKE, FAKE, None) == NULLP
    assert lib.msa_sparse_attn_decode_noalloc(*args1, FAKE, FAKE + 4, FAKE, None) == MISAL
    assert lib.msa_sparse_attn_decode_noalloc(ctypes.byref(_dims(head_dim=96)), ctypes.byref(c), ctypes.byref(b1.c),
                                              FAKE, FAKE, FAKE, None) == UNSUP


def test_decode_step_validates_on_the_host(lib):
    """msa_decode_step rejects what its four calls reject, before any HIP call."""
    d, c = _dims(), _cache()
    b2 = _Batch([1024, 900], [1, 2])
    b1 = _Batch([1024, 900], [1, 1])
    need = lib.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b1.c), 7)
    assert need >= lib.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(b1.c), 2)

    def call(b, ptrs=(FAKE,) * 5, ld=8, sel=FAKE, out=FAKE, ws=FAKE, nbytes=None, dims=d):
        return lib.msa_decode_step(ctypes.byref(dims), ctypes.byref(c), ctypes.byref(b.c), *ptrs[:4], ptrs[4], FAKE,
                                   ld, sel, out, ws, need if nbytes is None else nbytes, None)

    assert call(b2) == SHAPE                               # two queries in sequence 1
    assert call(b1, ptrs=(None, FAKE, FAKE, FAKE, FAKE)) == NULLP
    assert call(b1, ptrs=(FAKE, FAKE, FAKE + 4, FAKE, FAKE)) == MISAL
    assert call(b1, ld=7) == SHAPE                         # 8 blocks needed
    assert call(b1, sel=None) == NULLP
    assert call(b1, nbytes=need - 1) == WS
    assert call(b1, ws=None) == WS
    assert call(b1, dims=_dims(index_dim=48)) == UNSUP


def test_workspace_grows_with_queries(lib):
    d, c = _dims(), _cache(num_blocks=4096, mbps=1024)
    sizes = [lib.msa_workspace_size(ctypes.byref(d), ctypes.byref(c), ctypes.byref(_Batch([n], [n]).c), 1)
             for n in (128, 4096, 65536)]
    assert sizes[0] < sizes[1] < sizes[2]
    # fp16 partials of up to 15 non-local blocks per (row, head) dominate
    assert sizes[2] >= 65536 * 48 * 15 * 128 * 2


def test_quality_entry_points_validate_on_the_host(lib):
    d, c = _dims(), _cache()
    b = _Batch([1024, 900], [1, 1])
    dp, cp, bp = ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c)
    # block mass: null / misaligned pointers, negative counts, short rows
    # (the dense mass with sel NULL, the candidate mass with a selection)
    for sel in (None, FAKE):
        assert lib.msa_block_attn_mass(dp, cp, bp, None, sel, FAKE, 4, FAKE, 16, None) == NULLP
        assert lib.msa_block_attn_mass(dp, cp, bp, FAKE, sel, FAKE + 4, 4, FAKE, 16, None) == MISAL
        assert lib.msa_block_attn_mass(dp, cp, bp, FAKE, sel, FAKE, -1, FAKE, 16, None) == SHAPE
        assert lib.msa_block_attn_mass(dp, cp, bp, FAKE, sel, FAKE, 4, FAKE, 7, None) == SHAPE  # 8 blocks needed
        assert lib.msa_block_attn_mass(dp, cp, bp, FAKE, sel, FAKE, 0, FAKE, 16, None) == OK  # nothing to do
    assert lib.msa_block_attn_mass(dp, cp, bp, FAKE, FAKE + 8, FAKE, 4, FAKE, 16, None) == MISAL
    # selection quality
    assert lib.msa_selection_quality(dp, bp, FAKE, 4, FAKE, FAKE, FAKE, None, 16, FAKE, None) == NULLP
    assert lib.msa_selection_quality(dp, bp, FAKE, 4, FAKE, None, FAKE, FAKE, 16, FAKE, None) == NULLP
    assert lib.msa_selection_quality(dp, bp, FAKE, -2, FAKE, FAKE, FAKE, FAKE, 16, FAKE, None) == SHAPE
    assert lib.msa_selection_quality(dp, bp, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 3, FAKE, None) == SHAPE
    assert lib.msa_selection_quality(dp, bp, FAKE, 0, FAKE, FAKE, FAKE, FAKE, 16, FAKE, None) == OK


def test_dense_attention_validates_on_the_host(lib):
    d, c = _dims(), _cache()
    b = _Batch([1024, 900], [512, 3])
    dp, cp, bp = ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c)
    assert lib.msa_dense_attn_prefill(dp, cp, bp, None, FAKE, None) == NULLP
    assert lib.msa_dense_attn_prefill(dp, cp, bp, FAKE, FAKE + 2, None) == MISAL
    assert lib.msa_dense_attn_prefill(ctypes.byref(_dims(head_dim=96)), cp, bp, FAKE, FAKE, None) == UNSUP
    short = _cache(mbps=4)  # 1024 tokens need 8 blocks
    assert lib.msa_dense_attn_prefill(dp, ctypes.byref(short), bp, FAKE, FAKE, None) == CAP
    bad = _Batch([100], [101])  # more queries than tokens
    assert lib.msa_dense_attn_prefill(dp, cp, ctypes.byref(bad.c), FAKE, FAKE, None) == SHAPE
    empty = _Batch([100, 5], [0, 0])
    assert lib.msa_dense_attn_prefill(dp, cp, ctypes.byref(empty.c), FAKE, FAKE, None) == OK  # nothing to do


def test_dense_decode_validates_on_the_host(lib):
    d, c = _dims(), _cache()
    b = _Batch([1024, 900], [1, 1])
    dp, cp, bp = ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c)
    need = lib.msa_workspace_size(dp, cp, bp, 3)
    # 2 sequences x 8 groups x 1 split x 6 heads: fp32 rows of 128 dims plus one log-mass each
    assert need >= 2 * 8 * 6 * (128 + 1) * 4
    assert lib.msa_dense_attn_decode(dp, cp, bp, None, FAKE, FAKE, need, None) == NULLP
    assert lib.msa_dense_attn_decode(dp, cp, bp, FAKE, FAKE, FAKE, need - 1, None) == WS
    assert lib.msa_dense_attn_decode(dp, cp, bp, FAKE, FAKE, None, need, None) == WS
    assert lib.msa_dense_attn_decode(dp, cp, bp, FAKE, FAKE, FAKE + 8, need, None) == MISAL
    two = _Batch([1024, 900], [2, 1])  # decode takes one query per sequence
    assert lib.msa_dense_attn_decode(dp, cp, ctypes.byref(two.c), FAKE, FAKE, FAKE, need, None) == SHAPE
    # one partial per 64-block split of the context
    big = _cache(mbps=192)
    one = lib.msa_workspace_size(dp, ctypes.byref(big), ctypes.byref(_Batch([1024], [1]).c), 3)
    three = lib.msa_workspace_size(dp, ctypes.byref(big), ctypes.byref(_Batch([128 * 64 * 3], [1]).c), 3)
    assert 2.9 * one < three < 3.1 * one


def test_index_select_validates_on_the_host(lib):
    d, c = _dims(), _cache()
    b = _Batch([1024, 900], [300, 1])
    dp, cp, bp = ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c)
    need = lib.msa_workspace_size(dp, cp, bp, 4)
    # a 256-byte descriptor plus every row's pooled scores (Hkv x 8 blocks, fp32): the batch fits in one chunk
    assert need == 256 + 301 * 8 * 8 * 4
    one_row = 256 + 8 * 8 * 4
    assert lib.msa_index_select(dp, cp, bp, None, FAKE, FAKE, need, None) == NULLP
    assert lib.msa_index_select(dp, cp, bp, FAKE, None, FAKE, need, None) == NULLP
    assert lib.msa_index_select(dp, cp, bp, FAKE, FAKE, FAKE, one_row - 1, None) == WS
    assert lib.msa_index_select(dp, cp, bp, FAKE, FAKE, None, need, None) == WS
    assert lib.msa_index_select(dp, cp, bp, FAKE, FAKE, FAKE + 8, need, None) == MISAL
    empty = _Batch([100, 5], [0, 0])
    assert lib.msa_index_select(dp, cp, ctypes.byref(empty.c), FAKE, FAKE, FAKE, one_row, None) == OK
    # long batches are capped near 192 MB of pooled scores per chunk
    big_c = _cache(num_blocks=8192, mbps=8192)
    big = _Batch([1 << 20], [1 << 16])
    size = lib.msa_workspace_size(dp, ctypes.byref(big_c), ctypes.byref(big.c), 4)
    assert (192 << 20) - 8 * 8192 * 4 < size - 256 <= 192 << 20


def test_prefill_plan_and_run_validate_on_the_host(lib):
    d, c = _dims(), _cache()
    b = _Batch([1024, 900], [300, 2])
    dp, cp, bp = ctypes.byref(d), ctypes.byref(c), ctypes.byref(b.c)
    whole = lib.msa_workspace_size(dp, cp, bp, 1)
    plan = lib.msa_workspace_size(dp, cp, bp, 5)
    run = lib.msa_workspace_size(dp, cp, bp, 6)
    assert plan > 0 and run > 0 and plan + run == whole
    # plan(sel, plan, plan_bytes, stream): every call below fails before any launch
    assert lib.msa_sparse_attn_prefill_plan(dp, cp, bp, None, FAKE, plan, None) == NULLP
    assert lib.msa_sparse_attn_prefill_plan(dp, cp, bp, FAKE, None, plan, None) == WS
    assert lib.msa_sparse_attn_prefill_plan(dp, cp, bp, FAKE, FAKE, plan - 1, None) == WS
    assert lib.msa_sparse_attn_prefill_plan(dp, cp, bp, FAKE, FAKE + 8, plan, None) == MISAL
    # run(q, sel, plan, out, workspace, ws_bytes, stream)
    assert lib.msa_sparse_attn_prefill_run(dp, cp, bp, None, FAKE, FAKE, FAKE, FAKE, run, None) == NULLP
    assert lib.msa_sparse_attn_prefill_run(dp, cp, bp, FAKE, FAKE, None, FAKE, FAKE, run, None) == NULLP
    assert lib.msa_sparse_attn_prefill_run(dp, cp, bp, FAKE, FAKE, FAKE + 8, FAKE, FAKE, run, None) == MISAL
    assert lib.msa_sparse_attn_prefill_run(dp, cp, bp, FAKE, FAKE, FAKE, FAKE, FAKE, run - 1, None) == WS
    assert lib.msa_sparse_attn_prefill_run(dp, cp, bp, FAKE, FAKE, FAKE, FAKE, None, run, None) == WS
    # more blocks per sequence than one prefill call supports
    big = _cache(num_blocks=20000, mbps=20000)
    assert lib.msa_workspace_size(dp, ctypes.byref(big), bp, 5) == 0
    assert lib.msa_sparse_attn_prefill_plan(dp, ctypes.byref(big), bp, FAKE, FAKE, 1 << 30, None) == CAP
    assert lib.msa_sparse_attn_prefill_run(dp, ctypes.byref(big), bp, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                           None) == CAP


def test_prepare_checks_tensors_once_on_the_host(lib):
    """ops.prepare marshals a call's arguments up front: a wrong dtype or a
    non-contiguous tensor is refused when the call is prepared (nothing is
    launched here)."""
    import torch
    from block_sparse_long_score_amd import ops
    dims = ops.Dims(48, 8, 128, 64)
    batch = ops.Batch.make([300], [300], "cpu")
    scores = torch.zeros((300, 8, 3), dtype=torch.float32)
    sel = torch.zeros((300, 8, 16), dtype=torch.int32)
    call = ops.prepare("msa_block_topk", dims, batch, scores, sel)
    assert isinstance(call, ops.PreparedCall)
    with pytest.raises(TypeError):
        ops.prepare("msa_block_topk", dims, batch, scores.double(), sel)
    with pytest.raises(ValueError):
        ops.prepare("msa_block_topk", dims, batch, scores, sel.transpose(0, 1))
    with pytest.raises(KeyError):
        ops.prepare("msa_dense_attn_prefill", dims, batch, scores, sel)

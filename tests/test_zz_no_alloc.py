"""GPU: the allocation-free BlockMask build (flexattn_block_mask_build_noalloc) through the C ABI.

It must give the lists of flexattn_block_mask_build (which takes a caller workspace) bit for
bit, on two calls in a row whose second input is smaller (the static scratch keeps the first
call's summaries), and refuse, before enqueuing anything, a request whose summaries exceed its
static scratch.
"""
import ctypes

import numpy as np
import pytest

from workloads import random_case

pytestmark = pytest.mark.gpu

KEYS = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices", "row_order")


def _noalloc(fa, mk, B, Lq, Lkv, bq, bk, qd, kd, window, row_order, stream):
    from block_sparse_masked_blockmask_amd.flexattn import FaBlockMask, FaParams
    L = fa.lib()
    L.flexattn_block_mask_build_noalloc.argtypes = [ctypes.c_int, ctypes.POINTER(FaParams), ctypes.c_int,
                                                    ctypes.c_int, ctypes.c_int, ctypes.POINTER(FaBlockMask),
                                                    ctypes.c_void_p]
    L.flexattn_block_mask_build_noalloc.restype = ctypes.c_int
    import torch
    out = fa.BlockMask(B if (mk & fa.FA_MASK_DOC) else 1, 1, Lq, Lkv, bq, bk, torch.device("cuda", 0),
                       row_order=row_order)
    p = FaParams(0.0, window, 0, 0.0, None, None if qd is None else qd.data_ptr(),
                 None if kd is None else kd.data_ptr())
    s = out.as_struct()
    st = L.flexattn_block_mask_build_noalloc(mk, ctypes.byref(p), B, Lq, Lkv, ctypes.byref(s), stream.cuda_stream)
    return st, out


def _case(fa, torch, seed, B, L, bq, bk, mk, window=0, row_order=False, alias=True):
    dev = torch.device("cuda", 0)
    w = random_case(seed, dtype="bf16", B=B, Hq=1, Lq=L, D=8, doc=True, n_docs=max(2, L // 97))
    qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev) if mk & fa.FA_MASK_DOC else None
    kd = (qd if alias else qd.clone()) if qd is not None else None
    stream = torch.cuda.current_stream()
    ref = fa.flexattn_block_mask_build(mk, B, L, L, bq, bk, q_doc=qd, kv_doc=kd, window=window, row_order=row_order)
    st, got = _noalloc(fa, mk, B, L, L, bq, bk, qd, kd, window, row_order, stream)
    assert st == fa.FA_OK, fa.flexattn_last_error()
    torch.cuda.synchronize()
    for k in KEYS:
        a, b = getattr(got, k), getattr(ref, k)
        if a is None:
            assert b is None
            continue
        assert torch.equal(a, b), k


def test_noalloc_matches_workspace_build_twice_shrinking():
    import torch
    import block_sparse_masked_blockmask_amd as fa
    doc = fa.FA_MASK_DOC
    # Larger input first, then a smaller one: the scratch keeps the first call's summaries.
    _case(fa, torch, 1, 3, 20000, 128, 64, doc | fa.FA_MASK_CAUSAL, row_order=True)
    _case(fa, torch, 2, 2, 3000, 128, 128, doc | fa.FA_MASK_CAUSAL, alias=False)
    # Without DOC there is no scratch: the entry point reduces to the plain builder.
    _case(fa, torch, 3, 1, 5000, 128, 64, fa.FA_MASK_CAUSAL | fa.FA_MASK_WINDOW, window=700)
    _case(fa, torch, 4, 2, 900, 64, 64, doc)


def test_noalloc_refuses_beyond_its_scratch():
    import torch
    import block_sparse_masked_blockmask_amd as fa
    L = fa.lib()
    L.flexattn_block_mask_noalloc_max_bytes.restype = ctypes.c_size_t
    cap = L.flexattn_block_mask_noalloc_max_bytes()
    assert cap == 1 << 20
    # 16 bytes per block and side: 2 * 8192 blocks of 64 tokens per batch, 8 batches = 2 MiB.
    B, Lq = 8, 8192 * 64
    need = fa.flexattn_block_mask_workspace_bytes(fa.FA_MASK_DOC, B, Lq, Lq, 64, 64)
    assert need > cap
    dev = torch.device("cuda", 0)
    ids = torch.zeros((B, Lq), dtype=torch.int32, device=dev)
    from block_sparse_masked_blockmask_amd.flexattn import FaBlockMask, FaParams
    n = Lq // 64
    fake = FaBlockMask(B, 1, Lq, Lq, 64, 64, n, n, 4096, 4096, 4096, 4096, None)  # refused before any use
    p = FaParams(0.0, 0, 0, 0.0, None, ids.data_ptr(), ids.data_ptr())
    L.flexattn_block_mask_build_noalloc.argtypes = [ctypes.c_int, ctypes.POINTER(FaParams), ctypes.c_int,
                                                    ctypes.c_int, ctypes.c_int, ctypes.POINTER(FaBlockMask),
                                                    ctypes.c_void_p]
    L.flexattn_block_mask_build_noalloc.restype = ctypes.c_int
    st = L.flexattn_block_mask_build_noalloc(fa.FA_MASK_DOC, ctypes.byref(p), B, Lq, Lq, ctypes.byref(fake), None)
    assert st == fa.FA_ERR_UNSUPPORTED and "static scratch" in fa.flexattn_last_error()

"""CPU checks of the C ABI: the library loads, exports every declared entry point, sizes
are right, and argument validation rejects bad calls before anything is enqueued
(these calls return before any HIP API call, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_masked_blockmask_amd as fa
from block_sparse_masked_blockmask_amd.flexattn import FaBlockMask, FaParams, FaTensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flexattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flexattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 7
    lib = fa.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(flexattn_\w+)", out))
    assert set(names) <= exported, set(names) - exported


def test_struct_sizes_match_abi():
    # fa_tensor: ptr, 5 x int32, 3 x int64, ptr with natural alignment.
    assert ctypes.sizeof(FaTensor) == 8 + 4 * 5 + 4 + 8 * 3 + 8
    assert ctypes.sizeof(FaParams) == 4 * 4 + 8 * 3
    assert ctypes.sizeof(FaBlockMask) == 4 * 8 + 8 * 5  # four index arrays and the optional row_order


def test_sizes():
    assert fa.flexattn_block_mask_index_bytes(2, 1, 300, 200, 128, 64) == 2 * 3 * 4 * 4
    assert fa.flexattn_block_mask_count_bytes(2, 1, 300, 128) == 2 * 3 * 4
    assert fa.flexattn_block_mask_workspace_bytes(fa.FA_MASK_CAUSAL, 2, 300, 200, 128, 64) == 0
    assert fa.flexattn_block_mask_workspace_bytes(fa.FA_MASK_DOC, 2, 300, 200, 128, 64) == 2 * (3 + 4) * 16
    assert fa.flexattn_block_mask_index_bytes(0, 1, 10, 10, 128, 128) == 0
    assert fa.flexattn_version() >= 100


def _t(dtype=fa.FA_BF16, B=1, H=2, L=100, D=128, data=256):
    return FaTensor(data, dtype, B, H, L, D, H * L * D, L * D, D, None)


def _fwd(q, k, v, out, bm=None, mask=0, score=0, p=None):
    lib = fa.lib()
    p = p or FaParams(0.0, 0, 0, 0.0, None, None, None)
    return lib.flexattn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                            None if bm is None else ctypes.byref(bm), mask, score, ctypes.byref(p),
                            ctypes.byref(out), None, None)


@pytest.mark.parametrize("case,status,needle", [
    ("null", fa.FA_ERR_INVALID_ARG, "must not be NULL"),
    ("d64", fa.FA_ERR_UNSUPPORTED, "head dim"),
    ("gqa", fa.FA_ERR_INVALID_ARG, "multiple of Hkv"),
    ("dtype_mix", fa.FA_ERR_INVALID_ARG, "share one dtype"),
    ("i8", fa.FA_ERR_INVALID_ARG, "expected 3"),
    ("prefix_causal", fa.FA_ERR_INVALID_ARG, "PREFIX_LM"),
    ("no_bm", fa.FA_ERR_INVALID_ARG, "BlockMask is required"),
    ("misaligned", fa.FA_ERR_INVALID_ARG, "16-byte aligned"),
    ("stride", fa.FA_ERR_INVALID_ARG, "multiples of 8"),
    ("window0", fa.FA_ERR_INVALID_ARG, "window"),
    ("softcap0", fa.FA_ERR_INVALID_ARG, "softcap"),
    ("alibi_null", fa.FA_ERR_INVALID_ARG, "alibi"),
    ("bm_len", fa.FA_ERR_INVALID_ARG, "built for lengths"),
    ("bm_qblock", fa.FA_ERR_UNSUPPORTED, "q_block"),
    ("doc_null", fa.FA_ERR_INVALID_ARG, "q_doc"),
])
def test_fwd_validation(case, status, needle):
    q, k, v, o = _t(), _t(), _t(), _t()
    bm = None
    mask = score = 0
    p = None
    if case == "null":
        st = fa.lib().flexattn_fwd(None, None, None, None, 0, 0, None, None, None, None)
        assert st == status and needle in fa.flexattn_last_error()
        return
    if case == "d64":
        q, k, v, o = _t(D=64), _t(D=64), _t(D=64), _t(D=64)
    if case == "gqa":
        q, o = _t(H=3), _t(H=3)
    if case == "dtype_mix":
        k = _t(dtype=fa.FA_F32)
    if case == "i8":
        q, k, v, o = (_t(dtype=fa.FA_I8) for _ in range(4))
    if case == "prefix_causal":
        mask = fa.FA_MASK_PREFIX_LM | fa.FA_MASK_CAUSAL
        p = FaParams(0.0, 0, 4, 0.0, None, None, None)
    if case == "no_bm":
        mask = fa.FA_MASK_CAUSAL
    if case == "misaligned":
        q = _t(data=258)
    if case == "stride":
        q = FaTensor(256, fa.FA_BF16, 1, 2, 100, 128, 2 * 100 * 128, 100 * 130 + 4, 130, None)
    if case == "window0":
        mask = fa.FA_MASK_WINDOW
        bm = FaBlockMask(1, 1, 100, 100, 128, 128, 1, 1, 64, 64, 64, 64)
    if case == "softcap0":
        score = fa.FA_SCORE_SOFTCAP
    if case == "alibi_null":
        score = fa.FA_SCORE_ALIBI
    if case == "bm_len":
        mask = fa.FA_MASK_CAUSAL
        bm = FaBlockMask(1, 1, 90, 100, 128, 128, 1, 1, 64, 64, 64, 64)
    if case == "bm_qblock":
        mask = fa.FA_MASK_CAUSAL
        bm = FaBlockMask(1, 1, 100, 100, 64, 128, 2, 1, 64, 64, 64, 64)
    if case == "doc_null":
        mask = fa.FA_MASK_DOC
    st = _fwd(q, k, v, o, bm, mask, score, p)
    assert st == status, (st, fa.flexattn_last_error())
    assert needle in fa.flexattn_last_error(), fa.flexattn_last_error()


def test_block_mask_build_validation():
    lib = fa.lib()
    p = FaParams(0.0, 0, 0, 0.0, None, None, None)
    bm = FaBlockMask(1, 1, 100, 100, 128, 128, 1, 1, 64, 64, 64, 64)
    st = lib.flexattn_block_mask_build(fa.FA_MASK_CAUSAL, ctypes.byref(p), 1, 100, 120, ctypes.byref(bm), None, 0, None)
    assert st == fa.FA_ERR_INVALID_ARG and "kv_len" in fa.flexattn_last_error()
    bm2 = FaBlockMask(1, 1, 100, 100, 32, 128, 4, 1, 64, 64, 64, 64)
    st = lib.flexattn_block_mask_build(fa.FA_MASK_CAUSAL, ctypes.byref(p), 1, 100, 100, ctypes.byref(bm2), None, 0, None)
    assert st == fa.FA_ERR_UNSUPPORTED
    bm3 = FaBlockMask(1, 1, 100, 100, 128, 128, 1, 1, 64, 64, 64, 64)
    pd = FaParams(0.0, 0, 0, 0.0, None, 64, 64)
    st = lib.flexattn_block_mask_build(fa.FA_MASK_DOC, ctypes.byref(pd), 2, 100, 100, ctypes.byref(bm3), None, 0, None)
    assert st == fa.FA_ERR_INVALID_ARG and "Bm" in fa.flexattn_last_error()
    bm4 = FaBlockMask(2, 1, 100, 100, 128, 128, 1, 1, 64, 64, 64, 64)
    st = lib.flexattn_block_mask_build(fa.FA_MASK_DOC, ctypes.byref(pd), 2, 100, 100, ctypes.byref(bm4), None, 0, None)
    assert st == fa.FA_ERR_INVALID_ARG and "workspace" in fa.flexattn_last_error()
    st = lib.flexattn_block_mask_build(fa.FA_MASK_WINDOW, ctypes.byref(p), 1, 100, 100, ctypes.byref(bm), None, 0, None)
    assert st == fa.FA_ERR_INVALID_ARG and "window" in fa.flexattn_last_error()
    st = lib.flexattn_block_mask_build(64, ctypes.byref(p), 1, 100, 100, ctypes.byref(bm), None, 0, None)
    assert st == fa.FA_ERR_INVALID_ARG and "unknown" in fa.flexattn_last_error()
    # Misaligned arrays (including the optional schedule) are refused before anything runs.
    bm5 = FaBlockMask(1, 1, 100, 100, 128, 128, 1, 1, 64, 66, 64, 64)
    st = lib.flexattn_block_mask_build(fa.FA_MASK_CAUSAL, ctypes.byref(p), 1, 100, 100, ctypes.byref(bm5), None, 0, None)
    assert st == fa.FA_ERR_INVALID_ARG and "aligned" in fa.flexattn_last_error()
    bm6 = FaBlockMask(1, 1, 100, 100, 128, 128, 1, 1, 64, 64, 64, 64, 70)
    st = lib.flexattn_block_mask_build_host(fa.FA_MASK_CAUSAL, ctypes.byref(p), 1, 100, 100, ctypes.byref(bm6))
    assert st == fa.FA_ERR_INVALID_ARG and "aligned" in fa.flexattn_last_error()


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "block_sparse_masked_blockmask_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("oracles", ""), f


def test_quantize_validation():
    lib = fa.lib()
    q = _t()
    q8 = FaTensor(256, fa.FA_I8, 1, 2, 100, 128, 2 * 100 * 128, 100 * 128, 128, 512)
    v8 = FaTensor(256, fa.FA_FP8_E4M3, 1, 2, 100, 128, 2 * 100 * 128, 100 * 128, 128, 512)
    call = lambda *ts: lib.flexattn_quantize_qkv(*[ctypes.byref(t) for t in ts], None)
    bad = FaTensor(256, fa.FA_I8, 1, 2, 100, 128, 2 * 100 * 128, 100 * 128, 128, None)
    assert call(q, q, q, bad, q8, v8) == fa.FA_ERR_INVALID_ARG and "scale" in fa.flexattn_last_error()
    assert call(q, q, q, q8, q8, q8) == fa.FA_ERR_INVALID_ARG and "dtype" in fa.flexattn_last_error()
    d64 = FaTensor(256, fa.FA_BF16, 1, 2, 100, 64, 2 * 100 * 64, 100 * 64, 64, None)
    assert call(d64, q, q, q8, q8, v8) == fa.FA_ERR_UNSUPPORTED
    short = FaTensor(256, fa.FA_I8, 1, 2, 99, 128, 2 * 100 * 128, 100 * 128, 128, 512)
    assert call(q, q, q, short, q8, v8) == fa.FA_ERR_INVALID_ARG and "shapes" in fa.flexattn_last_error()


@pytest.mark.parametrize("case,status,needle", [
    ("splits0", fa.FA_ERR_INVALID_ARG, "n_splits"),
    ("splits_big", fa.FA_ERR_INVALID_ARG, "n_splits"),
    ("f32", fa.FA_ERR_UNSUPPORTED, "bf16"),
    ("no_ws", fa.FA_ERR_INVALID_ARG, "workspace needs"),
    ("ws_misaligned", fa.FA_ERR_INVALID_ARG, "16-byte aligned"),
    ("i8", fa.FA_ERR_UNSUPPORTED, "quantized"),
])
def test_splitkv_validation(case, status, needle):
    """flexattn_fwd_splitkv refuses before enqueuing anything (no GPU needed)."""
    lib = fa.lib()
    dt = {"f32": fa.FA_F32, "i8": fa.FA_I8}.get(case, fa.FA_BF16)
    q, k, v, o = _t(dtype=dt), _t(dtype=dt), _t(dtype=dt), _t(dtype=dt)
    p = FaParams(0.0, 0, 0, 0.0, None, None, None)
    n = {"splits0": 0, "splits_big": 257}.get(case, 4)
    need = lib.flexattn_fwd_splitkv_workspace_bytes(1, 2, 100, 4)
    assert need == 4 * 2 * 100 * 129 * 4
    ws, wsb = 4096, need
    if case == "no_ws":
        ws, wsb = None, 0
    if case == "ws_misaligned":
        ws = 4100
    st = lib.flexattn_fwd_splitkv(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None, 0, 0, ctypes.byref(p),
                                  ctypes.byref(o), None, n, ws, wsb, None)
    assert st == status, (st, fa.flexattn_last_error())
    assert needle in fa.flexattn_last_error(), fa.flexattn_last_error()


def test_bwd_sizes_and_struct():
    from block_sparse_masked_blockmask_amd.flexattn import FaBlockMaskTransposed
    assert ctypes.sizeof(FaBlockMaskTransposed) == 4 * 8 + 8 * 5  # four index arrays and the optional col_order
    rows4 = (2 * 3 * 130 + 3) // 4 * 4
    assert fa.flexattn_bwd_workspace_bytes(2, 3, 130) == (2 * rows4 + 2 * 3 * 2) * 4
    assert fa.flexattn_bwd_workspace_bytes(0, 3, 130) == 0


def _bm(Bm=1, Hm=1, Lq=100, Lkv=100, bq=128, bk=128, ptr=4096):
    nq, nk = -(-Lq // bq), -(-Lkv // bk)
    return FaBlockMask(Bm, Hm, Lq, Lkv, bq, bk, nq, nk, ptr, ptr, ptr, ptr)


def _bmt(Bm=1, Hm=1, Lq=100, Lkv=100, bq=128, bk=128, ptr=4096):
    from block_sparse_masked_blockmask_amd.flexattn import FaBlockMaskTransposed
    nq, nk = -(-Lq // bq), -(-Lkv // bk)
    return FaBlockMaskTransposed(Bm, Hm, Lq, Lkv, bq, bk, nq, nk, ptr, ptr, ptr, ptr)


@pytest.mark.parametrize("case,status,needle", [
    ("f32", fa.FA_ERR_UNSUPPORTED, "bf16"),
    ("d64", fa.FA_ERR_UNSUPPORTED, "head dim"),
    ("dk_shape", fa.FA_ERR_INVALID_ARG, "share one shape"),
    ("dq_shape", fa.FA_ERR_INVALID_ARG, "share one shape"),
    ("no_lse", fa.FA_ERR_INVALID_ARG, "lse is NULL"),
    ("mask_no_bm", fa.FA_ERR_INVALID_ARG, "BlockMask is required"),
    ("bm_only", fa.FA_ERR_INVALID_ARG, "both"),
    ("bm_64", fa.FA_ERR_UNSUPPORTED, "128 x 128"),
    ("bmt_dims", fa.FA_ERR_INVALID_ARG, "transposed"),
    ("dslopes_no_alibi", fa.FA_ERR_INVALID_ARG, "dslopes"),
    ("no_ws", fa.FA_ERR_INVALID_ARG, "workspace needs"),
    ("ws_misaligned", fa.FA_ERR_INVALID_ARG, "16-byte aligned"),
    ("gqa", fa.FA_ERR_INVALID_ARG, "multiple of Hkv"),
])
def test_bwd_validation(case, status, needle):
    """flexattn_bwd refuses before enqueuing anything (no GPU needed)."""
    lib = fa.lib()
    dt = fa.FA_F32 if case == "f32" else fa.FA_BF16
    D = 64 if case == "d64" else 128
    q, o, do, dq = (_t(dtype=dt, D=D) for _ in range(4))
    k, v = _t(dtype=dt, D=D), _t(dtype=dt, D=D)
    dk = _t(dtype=dt, D=D, L=90 if case == "dk_shape" else 100)
    dv = _t(dtype=dt, D=D)
    if case == "dq_shape":
        dq = _t(dtype=dt, D=D, H=4)
    if case == "gqa":
        k, v, dk, dv = (_t(H=3) for _ in range(4))
    p = FaParams(0.0, 0, 0, 0.0, None, None, None)
    lse = None if case == "no_lse" else 8192
    mask = fa.FA_MASK_CAUSAL if case in ("mask_no_bm", "bm_only", "bm_64", "bmt_dims") else 0
    bm = bmt = None
    if case in ("bm_only", "bm_64", "bmt_dims"):
        bm = _bm(bk=64 if case == "bm_64" else 128)
        if case != "bm_only":
            bmt = _bmt(bk=64 if case == "bm_64" else 128, Lkv=101 if case == "bmt_dims" else 100)
    dsl = 8192 if case == "dslopes_no_alibi" else None
    need = lib.flexattn_bwd_workspace_bytes(1, 2, 100)
    ws, wsb = 4096, need
    if case == "no_ws":
        ws, wsb = None, 0
    if case == "ws_misaligned":
        ws = 4100
    st = lib.flexattn_bwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o), ctypes.byref(do), lse,
                          None if bm is None else ctypes.byref(bm), None if bmt is None else ctypes.byref(bmt),
                          mask, 0, ctypes.byref(p), ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), dsl,
                          ws, wsb, None)
    assert st == status, (st, fa.flexattn_last_error())
    assert needle in fa.flexattn_last_error(), fa.flexattn_last_error()


def test_transpose_validation():
    lib = fa.lib()
    bm = _bm()
    for bad, needle in ((_bmt(Lq=101), "dimensions"), (_bmt(ptr=None), "NULL")):
        st = lib.flexattn_block_mask_transpose(ctypes.byref(bm), ctypes.byref(bad), None)
        assert st == fa.FA_ERR_INVALID_ARG and needle in fa.flexattn_last_error(), fa.flexattn_last_error()


def test_block_mask_and_fwd_workspace_sizes():
    # All four arrays: two counts [Bm][Hm][n_qb] and two index arrays [Bm][Hm][n_qb][n_kvb], int32.
    assert fa.flexattn_block_mask_bytes(2, 1, 300, 200, 128, 64) == 2 * (2 * 3 * 4 * 4) + 2 * (2 * 3 * 4)
    assert fa.flexattn_block_mask_bytes(1, 1, 134_449, 134_449, 128, 64) == \
        2 * fa.flexattn_block_mask_index_bytes(1, 1, 134_449, 134_449, 128, 64) + \
        2 * fa.flexattn_block_mask_count_bytes(1, 1, 134_449, 128)
    assert fa.flexattn_block_mask_bytes(0, 1, 10, 10, 128, 128) == 0
    assert fa.flexattn_block_mask_bytes(1, 1, 10, 10, 0, 128) == 0
    assert fa.flexattn_block_mask_bytes(1, 1, 0, 10, 128, 128) == 0   # no query block, no entry
    # The forward keeps every intermediate on chip: it needs no workspace in any form.
    lib = fa.lib()
    for dt in (fa.FA_BF16, fa.FA_F32, fa.FA_I8):
        q = _t(dtype=dt)
        for mask, score in ((0, 0), (fa.FA_MASK_DOC | fa.FA_MASK_CAUSAL, fa.FA_SCORE_SOFTCAP)):
            assert lib.flexattn_fwd_workspace_bytes(ctypes.byref(q), ctypes.byref(q), mask, score) == 0


def _arch_calls():
    """One argument-valid call of every entry point that enqueues work (fake, aligned device
    addresses: the calls are refused before any HIP call)."""
    lib = fa.lib()
    p = FaParams(0.0, 0, 0, 0.0, None, None, None)
    t = _t()
    q8 = FaTensor(256, fa.FA_I8, 1, 2, 100, 128, 2 * 100 * 128, 100 * 128, 128, 512)
    k8 = FaTensor(256, fa.FA_I8, 1, 2, 100, 128, 2 * 100 * 128, 100 * 128, 128, 512)
    v8 = FaTensor(256, fa.FA_FP8_E4M3, 1, 2, 100, 128, 2 * 100 * 128, 100 * 128, 128, 512)
    bm, bmt = _bm(), _bmt()
    r = lambda x: ctypes.byref(x)
    need_kv = lib.flexattn_fwd_splitkv_workspace_bytes(1, 2, 100, 4)
    need_b = lib.flexattn_bwd_workspace_bytes(1, 2, 100)
    return {
        "block_mask_build": lambda: lib.flexattn_block_mask_build(fa.FA_MASK_CAUSAL, r(p), 1, 100, 100, r(bm), None, 0,
                                                                  None),
        "fwd": lambda: lib.flexattn_fwd(r(t), r(t), r(t), r(bm), fa.FA_MASK_CAUSAL, 0, r(p), r(t), None, None),
        "fwd_nomask": lambda: lib.flexattn_fwd(r(t), r(t), r(t), None, 0, 0, r(p), r(t), 8192, None),
        "fwd_splitkv": lambda: lib.flexattn_fwd_splitkv(r(t), r(t), r(t), None, 0, 0, r(p), r(t), None, 4, 4096,
                                                        need_kv, None),
        "fwd_quantized": lambda: lib.flexattn_fwd(r(q8), r(k8), r(v8), None, 0, 0, r(p), r(t), None, None),
        "fwd_quant": lambda: lib.flexattn_fwd_quant(r(q8), r(k8), r(v8), 32, None, r(p), r(t), None, None),
        "quantize_qkv": lambda: lib.flexattn_quantize_qkv(r(t), r(t), r(t), r(q8), r(k8), r(v8), None),
        "quantize_qkv_ex": lambda: lib.flexattn_quantize_qkv_ex(r(t), r(t), r(t), r(q8), r(k8), r(v8), 128, None,
                                                                None, None, 0, None),
        "block_mask_transpose": lambda: lib.flexattn_block_mask_transpose(r(bm), r(bmt), None),
        "bwd": lambda: lib.flexattn_bwd(r(t), r(t), r(t), r(t), r(t), 8192, r(bm), r(bmt), fa.FA_MASK_CAUSAL, 0,
                                        r(p), r(t), r(t), r(t), None, 4096, need_b, None),
    }


@pytest.mark.parametrize("arch", ["gfx942:sramecc+:xnack-", "gfx90a", "gfx9500", "gfx95"])
@pytest.mark.parametrize("entry", sorted(_arch_calls()))
def test_non_gfx950_device_is_refused(monkeypatch, arch, entry):
    """Every entry point that enqueues work refuses another architecture with FA_ERR_UNSUPPORTED,
    naming it, after validating its arguments and before any HIP call (the device name is
    injected through FLEXATTN_DEVICE_ARCH)."""
    monkeypatch.setenv("FLEXATTN_DEVICE_ARCH", arch)
    st = _arch_calls()[entry]()
    assert st == fa.FA_ERR_UNSUPPORTED, (st, fa.flexattn_last_error())
    msg = fa.flexattn_last_error()
    assert arch in msg and "gfx950" in msg, msg
    # Invalid arguments still take precedence (validation first).
    lib = fa.lib()
    st = lib.flexattn_fwd(None, None, None, None, 0, 0, None, None, None, None)
    assert st == fa.FA_ERR_INVALID_ARG


def test_blockmask_clamp_helpers(tmp_path):
    """The clamps the kernels apply to caller-provided BlockMask counts and entries (host build of
    the shared header, with address and undefined-behaviour sanitizers)."""
    import shutil
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "clamp.cpp"
    src.write_text(r'''
#include "tile_class.h"
#include <cstdio>
#include <climits>
int main() {
  int bad = 0;
  const int cnt[][3] = {{-5, 7, 0}, {0, 7, 0}, {3, 7, 3}, {7, 7, 7}, {8, 7, 7}, {INT_MIN, 7, 0}, {INT_MAX, 7, 7},
                        {5, 0, 0}};
  for (auto& c : cnt) bad += fa::clamp_count(c[0], c[1]) != c[2];
  const int blk[][3] = {{-1, 10, 10}, {0, 10, 0}, {9, 10, 9}, {10, 10, 10}, {INT_MIN, 10, 10}, {INT_MAX, 10, 10},
                        {0, 0, 0}};
  for (auto& b : blk) bad += fa::sanitize_block(b[0], b[1]) != b[2];
  std::printf("%d\n", bad);
  return bad != 0;
}
''')
    exe = tmp_path / "clamp"
    r = subprocess.run([cxx, "-std=c++17", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
                        "-I" + os.path.join(ROOT, "block_sparse_masked_blockmask_amd", "csrc"), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stdout + r.stderr

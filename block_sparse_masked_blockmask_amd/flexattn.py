"""Python binding of libflexattn.so (ctypes): argument marshalling only.

Every entry point has the name of the C function it calls (include/flexattn.h) and only
turns torch tensors into the ABI's descriptors; all computation happens in the HIP kernels.
PyTorch provides device memory and the current stream. If the library is not built, every
call raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional

import torch

# FLEXATTN_LIBRARY selects another build of the same library (the tests load an
# address/undefined-behaviour-sanitized build of the host-side layer this way).
LIB_PATH = os.environ.get("FLEXATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                               "libflexattn.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_DEVICE = 0, 1, 2, 3
FA_F32, FA_BF16, FA_I8, FA_FP8_E4M3 = 0, 1, 2, 3
FA_MASK_NONE, FA_MASK_DOC, FA_MASK_CAUSAL, FA_MASK_WINDOW, FA_MASK_PREFIX_LM = 0, 1, 2, 4, 8
FA_SCORE_NONE, FA_SCORE_ALIBI, FA_SCORE_SOFTCAP = 0, 1, 2


class FaTensor(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("dtype", c_int32), ("B", c_int32), ("H", c_int32),
                ("L", c_int32), ("D", c_int32), ("stride_b", c_int64), ("stride_h", c_int64),
                ("stride_l", c_int64), ("scale", c_void_p)]


class FaParams(ctypes.Structure):
    _fields_ = [("sm_scale", c_float), ("window", c_int32), ("prefix_len", c_int32),
                ("softcap", c_float), ("alibi_slopes", c_void_p), ("q_doc", c_void_p),
                ("kv_doc", c_void_p)]


class FaBlockMask(ctypes.Structure):
    _fields_ = [("Bm", c_int32), ("Hm", c_int32), ("q_len", c_int32), ("kv_len", c_int32),
                ("q_block", c_int32), ("kv_block", c_int32), ("n_qb", c_int32), ("n_kvb", c_int32),
                ("kv_num_blocks", c_void_p), ("kv_indices", c_void_p),
                ("full_kv_num_blocks", c_void_p), ("full_kv_indices", c_void_p),
                ("row_order", c_void_p)]


class FaBlockMaskTransposed(ctypes.Structure):
    _fields_ = [("Bm", c_int32), ("Hm", c_int32), ("q_len", c_int32), ("kv_len", c_int32),
                ("q_block", c_int32), ("kv_block", c_int32), ("n_qb", c_int32), ("n_kvb", c_int32),
                ("q_num_blocks", c_void_p), ("q_indices", c_void_p),
                ("full_q_num_blocks", c_void_p), ("full_q_indices", c_void_p),
                ("col_order", c_void_p)]


class FlexAttnError(RuntimeError):
    def __init__(self, status: int, reason: str):
        super().__init__(f"flexattn status {status}: {reason}")
        self.status = status
        self.reason = reason


_lib = None


def lib() -> ctypes.CDLL:
    """Load libflexattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.flexattn_block_mask_bytes.argtypes = [c_int] * 6
        L.flexattn_block_mask_bytes.restype = c_size_t
        L.flexattn_fwd_workspace_bytes.argtypes = [c_void_p, c_void_p, c_int, c_int]
        L.flexattn_fwd_workspace_bytes.restype = c_size_t
        L.flexattn_block_mask_index_bytes.argtypes = [c_int] * 6
        L.flexattn_block_mask_index_bytes.restype = c_size_t
        L.flexattn_block_mask_count_bytes.argtypes = [c_int] * 4
        L.flexattn_block_mask_count_bytes.restype = c_size_t
        L.flexattn_block_mask_workspace_bytes.argtypes = [c_int] * 6
        L.flexattn_block_mask_workspace_bytes.restype = c_size_t
        L.flexattn_block_mask_build.argtypes = [c_int, POINTER(FaParams), c_int, c_int, c_int,
                                                POINTER(FaBlockMask), c_void_p, c_size_t, c_void_p]
        L.flexattn_block_mask_build.restype = c_int
        L.flexattn_block_mask_noalloc_max_bytes.argtypes = []
        L.flexattn_block_mask_noalloc_max_bytes.restype = c_size_t
        L.flexattn_block_mask_build_noalloc.argtypes = [c_int, POINTER(FaParams), c_int, c_int, c_int,
                                                        POINTER(FaBlockMask), c_void_p]
        L.flexattn_block_mask_build_noalloc.restype = c_int
        L.flexattn_block_mask_build_host.argtypes = [c_int, POINTER(FaParams), c_int, c_int, c_int,
                                                     POINTER(FaBlockMask)]
        L.flexattn_block_mask_build_host.restype = c_int
        L.flexattn_fwd.argtypes = [POINTER(FaTensor), POINTER(FaTensor), POINTER(FaTensor),
                                   POINTER(FaBlockMask), c_int, c_int, POINTER(FaParams),
                                   POINTER(FaTensor), c_void_p, c_void_p]
        L.flexattn_fwd.restype = c_int
        L.flexattn_fwd_splitkv_workspace_bytes.argtypes = [c_int] * 4
        L.flexattn_fwd_splitkv_workspace_bytes.restype = c_size_t
        L.flexattn_fwd_splitkv.argtypes = [POINTER(FaTensor), POINTER(FaTensor), POINTER(FaTensor),
                                           POINTER(FaBlockMask), c_int, c_int, POINTER(FaParams),
                                           POINTER(FaTensor), c_void_p, c_int, c_void_p, c_size_t, c_void_p]
        L.flexattn_fwd_splitkv.restype = c_int
        L.flexattn_quantize_qkv.argtypes = [POINTER(FaTensor)] * 6 + [c_void_p]
        L.flexattn_quantize_qkv_ex_workspace_bytes.argtypes = [c_int] * 3
        L.flexattn_quantize_qkv_ex_workspace_bytes.restype = c_size_t
        L.flexattn_quantize_qkv_ex.argtypes = [POINTER(FaTensor)] * 6 + [c_int, c_void_p, c_void_p, c_void_p,
                                                                          c_size_t, c_void_p]
        L.flexattn_quantize_qkv_ex.restype = c_int
        L.flexattn_fwd_quant.argtypes = [POINTER(FaTensor)] * 3 + [c_int, c_void_p, POINTER(FaParams),
                                                                   POINTER(FaTensor), c_void_p, c_void_p]
        L.flexattn_fwd_quant.restype = c_int
        L.flexattn_block_mask_transpose.argtypes = [POINTER(FaBlockMask), POINTER(FaBlockMaskTransposed), c_void_p]
        L.flexattn_block_mask_transpose.restype = c_int
        L.flexattn_bwd_workspace_bytes.argtypes = [c_int] * 3
        L.flexattn_bwd_workspace_bytes.restype = c_size_t
        L.flexattn_bwd.argtypes = [POINTER(FaTensor)] * 5 + [c_void_p, POINTER(FaBlockMask),
                                   POINTER(FaBlockMaskTransposed), c_int, c_int, POINTER(FaParams)] + \
                                  [POINTER(FaTensor)] * 3 + [c_void_p, c_void_p, c_size_t, c_void_p]
        L.flexattn_bwd.restype = c_int
        L.flexattn_quantize_qkv.restype = c_int
        L.flexattn_last_error.argtypes = []
        L.flexattn_last_error.restype = ctypes.c_char_p
        L.flexattn_version.argtypes = []
        L.flexattn_version.restype = c_int
        _lib = L
    return _lib


def flexattn_last_error() -> str:
    return lib().flexattn_last_error().decode()


def flexattn_version() -> int:
    return lib().flexattn_version()


def _check(status: int):
    if status != FA_OK:
        raise FlexAttnError(status, flexattn_last_error())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _record(stream, *tensors):
    """Tensors that this binding allocated (on the current stream) and handed to kernels on
    `stream`: record that use with the caching allocator, so that their memory is not given to
    another allocation on the current stream while those kernels may still run. Outputs and
    workspaces the caller passes in are the caller's to order."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            t.record_stream(s)


_DTYPES = {torch.float32: FA_F32, torch.bfloat16: FA_BF16, torch.int8: FA_I8, torch.uint8: FA_FP8_E4M3}
if hasattr(torch, "float8_e4m3fn"):
    _DTYPES[torch.float8_e4m3fn] = FA_FP8_E4M3


def tensor_desc(t: torch.Tensor, scale: Optional[torch.Tensor] = None) -> FaTensor:
    """Descriptor of a [B, H, L, D] tensor whose last dimension is contiguous."""
    if t.dim() != 4:
        raise ValueError("attention tensors are [B, H, L, D]")
    B, H, L, D = t.shape
    if t.numel() == 0:  # no element is addressed: describe it with the dense layout
        return FaTensor(t.data_ptr(), _DTYPES[t.dtype], B, H, L, D, H * L * D, L * D, D, _ptr(scale))
    if t.stride(3) != 1:
        raise ValueError("the D dimension must be contiguous")
    return FaTensor(t.data_ptr(), _DTYPES[t.dtype], B, H, L, D, t.stride(0), t.stride(1), t.stride(2),
                    _ptr(scale))


def flexattn_block_mask_bytes(Bm, Hm, q_len, kv_len, q_block, kv_block) -> int:
    return lib().flexattn_block_mask_bytes(Bm, Hm, q_len, kv_len, q_block, kv_block)


def flexattn_fwd_workspace_bytes(q: torch.Tensor, k: torch.Tensor, mask_kind: int = FA_MASK_NONE,
                                 score_kind: int = FA_SCORE_NONE) -> int:
    tq, tk = tensor_desc(q), tensor_desc(k)
    return lib().flexattn_fwd_workspace_bytes(ctypes.byref(tq), ctypes.byref(tk), mask_kind, score_kind)


def flexattn_block_mask_index_bytes(Bm, Hm, q_len, kv_len, q_block, kv_block) -> int:
    return lib().flexattn_block_mask_index_bytes(Bm, Hm, q_len, kv_len, q_block, kv_block)


def flexattn_block_mask_count_bytes(Bm, Hm, q_len, q_block) -> int:
    return lib().flexattn_block_mask_count_bytes(Bm, Hm, q_len, q_block)


def flexattn_block_mask_workspace_bytes(mask_kind, B, q_len, kv_len, q_block, kv_block) -> int:
    return lib().flexattn_block_mask_workspace_bytes(mask_kind, B, q_len, kv_len, q_block, kv_block)


class BlockMask:
    """Device BlockMask: the four int32 arrays plus their dimensions (caller-owned memory).

    row_order=True also allocates the optional schedule array (query blocks of each row set by
    decreasing cost), which the builders fill and the forward uses to start costly rows first."""

    def __init__(self, Bm, Hm, q_len, kv_len, q_block, kv_block, device, row_order: bool = False):
        self.Bm, self.Hm, self.q_len, self.kv_len = Bm, Hm, q_len, kv_len
        self.q_block, self.kv_block = q_block, kv_block
        self.n_qb = -(-q_len // q_block)
        self.n_kvb = -(-kv_len // kv_block)
        z = dict(dtype=torch.int32, device=device)
        self.kv_num_blocks = torch.empty((Bm, Hm, self.n_qb), **z)
        self.full_kv_num_blocks = torch.empty((Bm, Hm, self.n_qb), **z)
        self.kv_indices = torch.empty((Bm, Hm, self.n_qb, self.n_kvb), **z)
        self.full_kv_indices = torch.empty((Bm, Hm, self.n_qb, self.n_kvb), **z)
        self.row_order = torch.empty((Bm, Hm, self.n_qb), **z) if row_order else None

    def arrays(self):
        return [t for t in (self.kv_num_blocks, self.full_kv_num_blocks, self.kv_indices, self.full_kv_indices,
                            self.row_order) if t is not None]

    def to(self, device) -> "BlockMask":
        """A copy of this BlockMask with its arrays on `device`."""
        bm = BlockMask.__new__(BlockMask)
        bm.__dict__.update(self.__dict__)
        for k in ("kv_num_blocks", "full_kv_num_blocks", "kv_indices", "full_kv_indices", "row_order"):
            if getattr(self, k) is not None:
                setattr(bm, k, getattr(self, k).to(device))
        return bm

    def as_struct(self) -> FaBlockMask:
        return FaBlockMask(self.Bm, self.Hm, self.q_len, self.kv_len, self.q_block, self.kv_block,
                           self.n_qb, self.n_kvb, self.kv_num_blocks.data_ptr(), self.kv_indices.data_ptr(),
                           self.full_kv_num_blocks.data_ptr(), self.full_kv_indices.data_ptr(),
                           _ptr(getattr(self, "row_order", None)))


def _params(window=0, prefix_len=0, softcap=0.0, alibi_slopes=None, q_doc=None, kv_doc=None, sm_scale=0.0):
    return FaParams(float(sm_scale), int(window), int(prefix_len), float(softcap), _ptr(alibi_slopes),
                    _ptr(q_doc), _ptr(kv_doc))


def flexattn_block_mask_build(mask_kind: int, B: int, q_len: int, kv_len: int, q_block: int = 128,
                              kv_block: int = 128, *, q_doc=None, kv_doc=None, window: int = 0,
                              prefix_len: int = 0, device=None, stream=None, out: Optional[BlockMask] = None,
                              workspace: Optional[torch.Tensor] = None, row_order: bool = False) -> BlockMask:
    """Build a BlockMask on the device (create_block_mask of the FlexAttention guide).
    row_order=True (with out=None) also computes the schedule array; with `out`, the schedule is
    computed when out.row_order is allocated."""
    if device is None:
        device = q_doc.device if q_doc is not None else torch.device("cuda", torch.cuda.current_device())
    tmp = []
    if out is None:
        Bm = B if (mask_kind & FA_MASK_DOC) else 1
        out = BlockMask(Bm, 1, q_len, kv_len, q_block, kv_block, device, row_order=row_order)
        tmp += out.arrays()
    ws_bytes = flexattn_block_mask_workspace_bytes(mask_kind, B, q_len, kv_len, q_block, kv_block)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        tmp.append(workspace)
    p = _params(window=window, prefix_len=prefix_len, q_doc=q_doc, kv_doc=kv_doc)
    s = out.as_struct()
    _check(lib().flexattn_block_mask_build(mask_kind, ctypes.byref(p), B, q_len, kv_len, ctypes.byref(s),
                                           _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                           _stream(stream)))
    _record(stream, *tmp)
    return out


def flexattn_block_mask_noalloc_max_bytes() -> int:
    return lib().flexattn_block_mask_noalloc_max_bytes()


def flexattn_block_mask_build_noalloc(mask_kind: int, B: int, q_len: int, kv_len: int, out: BlockMask, *,
                                      q_doc=None, kv_doc=None, window: int = 0, prefix_len: int = 0,
                                      stream=None) -> BlockMask:
    """Build a BlockMask into the caller's `out` with the allocation-free entry point (its scratch
    is a static device array; nothing is allocated by the library or here)."""
    p = _params(window=window, prefix_len=prefix_len, q_doc=q_doc, kv_doc=kv_doc)
    s = out.as_struct()
    _check(lib().flexattn_block_mask_build_noalloc(mask_kind, ctypes.byref(p), B, q_len, kv_len, ctypes.byref(s),
                                                   _stream(stream)))
    return out


def block_mask_all_partial(Bm: int, Hm: int, q_len: int, kv_len: int, q_block: int = 128, kv_block: int = 128,
                           device=None) -> BlockMask:
    """A BlockMask that lists every tile as partial: the kernel visits all tiles and evaluates the
    mask on every score (the dense-iteration baseline for a block-sparse BlockMask; both give the
    same result for the same mask)."""
    bm = BlockMask(Bm, Hm, q_len, kv_len, q_block, kv_block, device)
    bm.kv_num_blocks.fill_(bm.n_kvb)
    bm.full_kv_num_blocks.zero_()
    bm.kv_indices.copy_(torch.arange(bm.n_kvb, dtype=torch.int32, device=bm.kv_indices.device)
                        .expand_as(bm.kv_indices))
    bm.full_kv_indices.zero_()
    return bm


def flexattn_block_mask_build_host(mask_kind: int, B: int, q_len: int, kv_len: int, q_block: int = 128,
                                   kv_block: int = 128, *, q_doc=None, kv_doc=None, window: int = 0,
                                   prefix_len: int = 0, row_order: bool = False) -> BlockMask:
    """Build a BlockMask on the host: document ids and the returned arrays are CPU memory.
    row_order=True also computes the schedule array (as the device builder does)."""
    def host_ids(x):
        if x is None:
            return None
        t = x if isinstance(x, torch.Tensor) else torch.from_numpy(x)
        if t.device.type != "cpu" or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("document ids must be contiguous int32 CPU arrays")
        return t
    qd, kd = host_ids(q_doc), host_ids(kv_doc)
    Bm = B if (mask_kind & FA_MASK_DOC) else 1
    out = BlockMask(Bm, 1, q_len, kv_len, q_block, kv_block, torch.device("cpu"), row_order=row_order)
    p = _params(window=window, prefix_len=prefix_len, q_doc=qd, kv_doc=kd)
    s = out.as_struct()
    _check(lib().flexattn_block_mask_build_host(mask_kind, ctypes.byref(p), B, q_len, kv_len, ctypes.byref(s)))
    return out


def flexattn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: Optional[BlockMask] = None,
                 mask_kind: int = FA_MASK_NONE, score_kind: int = FA_SCORE_NONE, *, window: int = 0,
                 prefix_len: int = 0, softcap: float = 0.0, alibi_slopes=None, q_doc=None, kv_doc=None,
                 sm_scale: float = 0.0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 return_lse: bool = True, stream=None, q_scale=None, k_scale=None, v_scale=None):
    """Forward pass; returns (out, lse). lse is None when return_lse is False and none is given.

    For the quantized form pass the int8 q/k and E4M3 v codes with their scale arrays (as
    returned by flexattn_quantize_qkv); out is then bf16.
    """
    tmp = []
    if out is None:
        odt = torch.bfloat16 if q.dtype == torch.int8 else q.dtype
        out = torch.empty(q.shape, dtype=odt, device=q.device)
        tmp.append(out)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        tmp.append(lse)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3])):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Lq] tensor")
    tq, tk, tv, to = tensor_desc(q, q_scale), tensor_desc(k, k_scale), tensor_desc(v, v_scale), tensor_desc(out)
    p = _params(window=window, prefix_len=prefix_len, softcap=softcap, alibi_slopes=alibi_slopes,
                q_doc=q_doc, kv_doc=kv_doc, sm_scale=sm_scale)
    bm = ctypes.byref(block_mask.as_struct()) if block_mask is not None else None
    _check(lib().flexattn_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), bm, mask_kind, score_kind,
                              ctypes.byref(p), ctypes.byref(to), _ptr(lse), _stream(stream)))
    _record(stream, *tmp)
    return out, lse


def flexattn_fwd_splitkv_workspace_bytes(B: int, Hq: int, Lq: int, n_splits: int) -> int:
    return lib().flexattn_fwd_splitkv_workspace_bytes(B, Hq, Lq, n_splits)


def flexattn_fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: Optional[BlockMask] = None,
                         mask_kind: int = FA_MASK_NONE, score_kind: int = FA_SCORE_NONE, *, n_splits: int,
                         workspace: Optional[torch.Tensor] = None, window: int = 0, prefix_len: int = 0,
                         softcap: float = 0.0, alibi_slopes=None, q_doc=None, kv_doc=None, sm_scale: float = 0.0,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         return_lse: bool = True, stream=None):
    """Split-KV forward (flexattn_fwd_splitkv); returns (out, lse). The workspace is allocated
    when not given (flexattn_fwd_splitkv_workspace_bytes bytes)."""
    tmp = []
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
        tmp.append(out)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        tmp.append(lse)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3])):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Lq] tensor")
    ws_bytes = flexattn_fwd_splitkv_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], n_splits) if n_splits > 1 else 0
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        tmp.append(workspace)
    tq, tk, tv, to = tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(out)
    p = _params(window=window, prefix_len=prefix_len, softcap=softcap, alibi_slopes=alibi_slopes,
                q_doc=q_doc, kv_doc=kv_doc, sm_scale=sm_scale)
    bm = ctypes.byref(block_mask.as_struct()) if block_mask is not None else None
    _check(lib().flexattn_fwd_splitkv(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), bm, mask_kind,
                                      score_kind, ctypes.byref(p), ctypes.byref(to), _ptr(lse), n_splits,
                                      _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                      _stream(stream)))
    _record(stream, *tmp)
    return out, lse


def flexattn_quantize_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, out=None, stream=None):
    """Quantize bf16 q, k, v (flexattn_quantize_qkv). Returns a dict with q8, k8 (int8), v8
    (uint8 E4M3 codes) and their float32 scales q_scale [B,H,ceil(L/128)], k_scale, v_scale
    [B,H,128]; `out` may supply these tensors (same keys) to avoid allocation."""
    def blocks(t):
        return -(-t.shape[2] // 128)
    fresh = out is None
    if out is None:
        out = {
            "q8": torch.empty(q.shape, dtype=torch.int8, device=q.device),
            "k8": torch.empty(k.shape, dtype=torch.int8, device=k.device),
            "v8": torch.empty(v.shape, dtype=torch.uint8, device=v.device),
            "q_scale": torch.empty((q.shape[0], q.shape[1], blocks(q)), dtype=torch.float32, device=q.device),
            "k_scale": torch.empty((k.shape[0], k.shape[1], blocks(k)), dtype=torch.float32, device=k.device),
            "v_scale": torch.empty((v.shape[0], v.shape[1], v.shape[3]), dtype=torch.float32, device=v.device),
        }
    descs = [tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(out["q8"], out["q_scale"]),
             tensor_desc(out["k8"], out["k_scale"]), tensor_desc(out["v8"], out["v_scale"])]
    _check(lib().flexattn_quantize_qkv(*[ctypes.byref(d) for d in descs], _stream(stream)))
    if fresh:
        _record(stream, *out.values())
    return out


def flexattn_quantize_qkv_ex_workspace_bytes(B: int, Hkv: int, Lkv: int) -> int:
    return lib().flexattn_quantize_qkv_ex_workspace_bytes(B, Hkv, Lkv)


def flexattn_quantize_qkv_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, qk_block: int = 32,
                             center_k: bool = True, out=None, workspace=None, stream=None):
    """Quantize with the refinements (flexattn_quantize_qkv_ex): qk_block tokens per Q/K scale and,
    with center_k, K centering. Returns the dict of flexattn_quantize_qkv plus "qk_block", and with
    centering "k_mean" [B,Hkv,128] and "q_delta" [B,Hq,Lq] (float32)."""
    def blocks(t):
        return -(-t.shape[2] // qk_block)
    fresh = out is None
    if out is None:
        out = {
            "q8": torch.empty(q.shape, dtype=torch.int8, device=q.device),
            "k8": torch.empty(k.shape, dtype=torch.int8, device=k.device),
            "v8": torch.empty(v.shape, dtype=torch.uint8, device=v.device),
            "q_scale": torch.empty((q.shape[0], q.shape[1], blocks(q)), dtype=torch.float32, device=q.device),
            "k_scale": torch.empty((k.shape[0], k.shape[1], blocks(k)), dtype=torch.float32, device=k.device),
            "v_scale": torch.empty((v.shape[0], v.shape[1], v.shape[3]), dtype=torch.float32, device=v.device),
        }
        if center_k:
            out["k_mean"] = torch.empty((k.shape[0], k.shape[1], k.shape[3]), dtype=torch.float32, device=k.device)
            out["q_delta"] = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    out["qk_block"] = qk_block
    ws_bytes = flexattn_quantize_qkv_ex_workspace_bytes(k.shape[0], k.shape[1], k.shape[2]) if center_k else 0
    tmp = []
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        tmp.append(workspace)
    descs = [tensor_desc(q), tensor_desc(k), tensor_desc(v), tensor_desc(out["q8"], out["q_scale"]),
             tensor_desc(out["k8"], out["k_scale"]), tensor_desc(out["v8"], out["v_scale"])]
    _check(lib().flexattn_quantize_qkv_ex(*[ctypes.byref(d) for d in descs], qk_block,
                                          _ptr(out.get("k_mean") if center_k else None),
                                          _ptr(out.get("q_delta") if center_k else None), _ptr(workspace),
                                          workspace.numel() if workspace is not None else 0, _stream(stream)))
    _record(stream, *tmp, *(out.values() if fresh else ()))
    return out


def flexattn_fwd_quant(qz: dict, *, sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, return_lse: bool = True, stream=None):
    """Quantized forward (flexattn_fwd_quant) on the dict returned by flexattn_quantize_qkv_ex
    (or flexattn_quantize_qkv, qk_block 128); returns (out bf16, lse)."""
    q8 = qz["q8"]
    tmp = []
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
        tmp.append(out)
    if lse is None and return_lse:
        lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
        tmp.append(lse)
    tq, tk = tensor_desc(q8, qz["q_scale"]), tensor_desc(qz["k8"], qz["k_scale"])
    tv, to = tensor_desc(qz["v8"], qz["v_scale"]), tensor_desc(out)
    p = _params(sm_scale=sm_scale)
    _check(lib().flexattn_fwd_quant(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), qz.get("qk_block", 128),
                                    _ptr(qz.get("q_delta")), ctypes.byref(p), ctypes.byref(to), _ptr(lse),
                                    _stream(stream)))
    _record(stream, *tmp)
    return out, lse


class BlockMaskTransposed:
    """Device column view of a BlockMask (q-block lists per kv block; caller-owned memory).
    col_order=True also allocates the optional column schedule (kv blocks by decreasing cost),
    which the transpose fills and the backward's dk/dv pass uses."""

    def __init__(self, bm: BlockMask, col_order: bool = False):
        self.Bm, self.Hm, self.q_len, self.kv_len = bm.Bm, bm.Hm, bm.q_len, bm.kv_len
        self.q_block, self.kv_block, self.n_qb, self.n_kvb = bm.q_block, bm.kv_block, bm.n_qb, bm.n_kvb
        z = dict(dtype=torch.int32, device=bm.kv_num_blocks.device)
        self.q_num_blocks = torch.empty((self.Bm, self.Hm, self.n_kvb), **z)
        self.full_q_num_blocks = torch.empty((self.Bm, self.Hm, self.n_kvb), **z)
        self.q_indices = torch.empty((self.Bm, self.Hm, self.n_kvb, self.n_qb), **z)
        self.full_q_indices = torch.empty((self.Bm, self.Hm, self.n_kvb, self.n_qb), **z)
        self.col_order = torch.empty((self.Bm, self.Hm, self.n_kvb), **z) if col_order else None

    def arrays(self):
        return [t for t in (self.q_num_blocks, self.full_q_num_blocks, self.q_indices, self.full_q_indices,
                            self.col_order) if t is not None]

    def as_struct(self) -> FaBlockMaskTransposed:
        return FaBlockMaskTransposed(self.Bm, self.Hm, self.q_len, self.kv_len, self.q_block, self.kv_block,
                                     self.n_qb, self.n_kvb, self.q_num_blocks.data_ptr(), self.q_indices.data_ptr(),
                                     self.full_q_num_blocks.data_ptr(), self.full_q_indices.data_ptr(),
                                     _ptr(self.col_order))


def flexattn_block_mask_transpose(block_mask: BlockMask, *, out: Optional[BlockMaskTransposed] = None,
                                  stream=None, col_order: bool = False) -> BlockMaskTransposed:
    """Column view of a device BlockMask (flexattn_block_mask_transpose); col_order=True (with
    out=None) also computes the column schedule."""
    fresh = out is None
    if out is None:
        out = BlockMaskTransposed(block_mask, col_order=col_order)
    s, t = block_mask.as_struct(), out.as_struct()
    _check(lib().flexattn_block_mask_transpose(ctypes.byref(s), ctypes.byref(t), _stream(stream)))
    if fresh:
        _record(stream, *out.arrays())
    return out


def flexattn_bwd_workspace_bytes(B: int, Hq: int, Lq: int) -> int:
    return lib().flexattn_bwd_workspace_bytes(B, Hq, Lq)


def flexattn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                 lse: torch.Tensor, block_mask: Optional[BlockMask] = None,
                 block_mask_t: Optional[BlockMaskTransposed] = None, mask_kind: int = FA_MASK_NONE,
                 score_kind: int = FA_SCORE_NONE, *, window: int = 0, prefix_len: int = 0, softcap: float = 0.0,
                 alibi_slopes=None, q_doc=None, kv_doc=None, sm_scale: float = 0.0, slope_grad: bool = False,
                 dq=None, dk=None, dv=None, dslopes=None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward pass (flexattn_bwd); returns (dq, dk, dv, dslopes). The transposed BlockMask is built
    when a BlockMask is given without one; dslopes is computed when slope_grad is set (ALiBi)."""
    tmp = []
    if block_mask is not None and block_mask_t is None:
        block_mask_t = flexattn_block_mask_transpose(block_mask, stream=stream)
        tmp += block_mask_t.arrays()
    if dq is None:
        dq = torch.empty(q.shape, dtype=q.dtype, device=q.device)
        tmp.append(dq)
    if dk is None:
        dk = torch.empty(k.shape, dtype=k.dtype, device=k.device)
        tmp.append(dk)
    if dv is None:
        dv = torch.empty(v.shape, dtype=v.dtype, device=v.device)
        tmp.append(dv)
    if slope_grad and dslopes is None:
        dslopes = torch.empty(q.shape[1], dtype=torch.float32, device=q.device)
        tmp.append(dslopes)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Lq] tensor")
    ws_bytes = flexattn_bwd_workspace_bytes(q.shape[0], q.shape[1], q.shape[2])
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        tmp.append(workspace)
    descs = [tensor_desc(t) for t in (q, k, v, out, dout, dq, dk, dv)]
    p = _params(window=window, prefix_len=prefix_len, softcap=softcap, alibi_slopes=alibi_slopes,
                q_doc=q_doc, kv_doc=kv_doc, sm_scale=sm_scale)
    bm = ctypes.byref(block_mask.as_struct()) if block_mask is not None else None
    bmt = ctypes.byref(block_mask_t.as_struct()) if block_mask_t is not None else None
    _check(lib().flexattn_bwd(*[ctypes.byref(d) for d in descs[:5]], _ptr(lse), bm, bmt, mask_kind, score_kind,
                              ctypes.byref(p), *[ctypes.byref(d) for d in descs[5:]], _ptr(dslopes),
                              _ptr(workspace), workspace.numel() if workspace is not None else 0,
                              _stream(stream)))
    _record(stream, *tmp)
    return dq, dk, dv, dslopes

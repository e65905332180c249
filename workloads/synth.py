"""Seeded workload generators (structure + Q/K/V); no attention arithmetic here."""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16. Inputs here are finite normals
    from `standard_normal`, so NaN handling is not needed; it is asserted.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert np.isfinite(x).all()
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


@dataclass
class Workload:
    """One synthetic attention problem.

    q, k, v are float32 arrays [B, H, L, D] for fp32 problems and uint16 bf16
    bit patterns for bf16 problems. The mask/score description is plain data.
    """
    name: str
    dtype: str                     # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lkv: int
    D: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    doc: bool = False
    causal: bool = False
    window: Optional[int] = None   # q - kv < window
    prefix_len: Optional[int] = None
    softcap: Optional[float] = None
    alibi_slopes: Optional[np.ndarray] = None  # float32 [Hq]
    q_doc: Optional[np.ndarray] = None          # int32 [B, Lq]
    kv_doc: Optional[np.ndarray] = None         # int32 [B, Lkv]
    v_channel_scale: Optional[np.ndarray] = None  # float32 [Hkv, D] (data property)
    meta: dict = field(default_factory=dict)

    def qkv_f32(self):
        """Q, K, V widened to float32 (exact for bf16 inputs)."""
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.q), bf16_bits_to_f32(self.k), bf16_bits_to_f32(self.v)
        return self.q, self.k, self.v


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _qkv(rng, B, Hq, Hkv, Lq, Lkv, D, dtype):
    q = _normal(rng, (B, Hq, Lq, D), dtype)
    k = _normal(rng, (B, Hkv, Lkv, D), dtype)
    v = _normal(rng, (B, Hkv, Lkv, D), dtype)
    return q, k, v


def group_ids(sizes) -> np.ndarray:
    """Packed group ids: group g occupies sizes[g] consecutive tokens."""
    return np.repeat(np.arange(len(sizes), dtype=np.int32), np.asarray(sizes))


def _tirex_small():
    """Four groups of 17 variates (1 target + 16 covariates), fp32, H=4, D=128."""
    rng = np.random.default_rng(1)
    doc = group_ids([17, 17, 17, 17])[None, :]
    L = doc.shape[1]
    q, k, v = _qkv(rng, 1, 4, 4, L, L, 128, "f32")
    return Workload("grouped_variate_4x17_f32", "f32", 1, 4, 4, L, L, 128, q, k, v,
                    doc=True, q_doc=doc, kv_doc=doc)


def _tirex_scale(with_tensors=True):
    """4096 groups with sizes uniform in [2, 64], packed without alignment; bf16."""
    rng = np.random.default_rng(2)
    sizes = rng.integers(2, 65, 4096)
    doc = group_ids(sizes)[None, :]
    L = doc.shape[1]
    if with_tensors:
        q, k, v = _qkv(rng, 1, 4, 4, L, L, 128, "bf16")
    else:
        q = k = v = None
    return Workload("grouped_variate_4096g_bf16", "bf16", 1, 4, 4, L, L, 128, q, k, v,
                    doc=True, q_doc=doc, kv_doc=doc, meta={"group_sizes": sizes})


def _doc_causal(with_tensors=True):
    """Causal document packing: per sequence, geometric(mean 512) lengths until T."""
    rng = np.random.default_rng(3)
    B, H, T = 4, 16, 8192
    docs = np.empty((B, T), dtype=np.int32)
    for b in range(B):
        pos, d = 0, 0
        while pos < T:
            n = int(rng.geometric(1.0 / 512))
            n = min(n, T - pos)
            docs[b, pos:pos + n] = d
            pos += n
            d += 1
    if with_tensors:
        q, k, v = _qkv(rng, B, H, H, T, T, 128, "bf16")
    else:
        q = k = v = None
    return Workload("doc_causal_b4h16t8192_bf16", "bf16", B, H, H, T, T, 128, q, k, v,
                    doc=True, causal=True, q_doc=docs, kv_doc=docs)


def _swa_gqa(with_tensors=True):
    """Sliding-window (1024) causal GQA 32/8 with soft-cap 50, T=16384, bf16."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, T = 2, 32, 8, 16384
    if with_tensors:
        q, k, v = _qkv(rng, B, Hq, Hkv, T, T, 128, "bf16")
    else:
        q = k = v = None
    return Workload("swa1024_gqa32x8_softcap50_t16384_bf16", "bf16", B, Hq, Hkv, T, T, 128,
                    q, k, v, causal=True, window=1024, softcap=50.0)


def _dense_long(with_tensors=True):
    """Dense self-attention, B=1, H=32, S=24576; V has per-channel scale U(0.5, 2)."""
    rng = np.random.default_rng(5)
    B, H, S, D = 1, 32, 24576, 128
    if with_tensors:
        q = _normal(rng, (B, H, S, D), "f32")
        k = _normal(rng, (B, H, S, D), "f32")
        v = _normal(rng, (B, H, S, D), "f32")
        s = rng.uniform(0.5, 2.0, size=(H, D)).astype(np.float32)
        v = v * s[None, :, None, :]
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    else:
        q = k = v = None
        s = None
    return Workload("dense_b1h32s24576_bf16", "bf16", B, H, H, S, S, D, q, k, v,
                    v_channel_scale=s)


def grouped_sweep(n_groups: int, dtype: str) -> Workload:
    """n_groups groups of 17 variates packed in order (TiRex2 shape: 1 target + 16 covariates),
    B=1, H=4, D=128; the group-count sweep of the grouped variate workload."""
    rng = np.random.default_rng(1000 + 2 * n_groups + (dtype == "bf16"))
    doc = group_ids([17] * n_groups)[None, :]
    L = doc.shape[1]
    q, k, v = _qkv(rng, 1, 4, 4, L, L, 128, dtype)
    return Workload(f"grouped_variate_{n_groups}x17_{dtype}", dtype, 1, 4, 4, L, L, 128, q, k, v,
                    doc=True, q_doc=doc, kv_doc=doc)


SWEEP_GROUPS = (8, 32, 64, 128)


def decode_workload() -> Workload:
    """Decoding shape: 16 new queries per sequence against 32768 cached keys, B=8, GQA 32/8,
    D=128, bf16, no mask (the split-KV form's workload)."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, Lq, Lkv = 8, 32, 8, 16, 32768
    q, k, v = _qkv(rng, B, Hq, Hkv, Lq, Lkv, 128, "bf16")
    return Workload("decode_b8h32x8_q16_kv32768_bf16", "bf16", B, Hq, Hkv, Lq, Lkv, 128, q, k, v)

WORKLOADS = {
    "grouped_variate_4x17_f32": _tirex_small,
    "grouped_variate_4096g_bf16": _tirex_scale,
    "doc_causal_b4h16t8192_bf16": _doc_causal,
    "swa1024_gqa32x8_softcap50_t16384_bf16": _swa_gqa,
    "dense_b1h32s24576_bf16": _dense_long,
}


def make_workload(name: str, with_tensors: bool = True) -> Workload:
    fn = WORKLOADS[name]
    if name == "grouped_variate_4x17_f32":
        return fn()
    return fn(with_tensors)


def random_case(seed: int, *, dtype="bf16", B=1, Hq=2, Hkv=None, Lq=200, Lkv=None, D=128,
                doc=False, causal=False, window=None, prefix_len=None, softcap=None,
                alibi=False, n_docs=None, doc_sorted=True) -> Workload:
    """A small seeded case for parity sweeps (ragged lengths, Lq != Lkv, GQA).

    Document ids are drawn as sorted runs (packing) or, with doc_sorted=False,
    independently per token (unsorted ids exercise the exhaustive path).
    """
    rng = np.random.default_rng(seed)
    Hkv = Hq if Hkv is None else Hkv
    Lkv = Lq if Lkv is None else Lkv
    q_doc = kv_doc = None
    if doc:
        n_docs = n_docs or max(1, Lq // 40)
        if doc_sorted:
            def runs(L):
                cuts = np.sort(rng.choice(np.arange(1, L), size=min(n_docs - 1, L - 1), replace=False)) \
                    if n_docs > 1 and L > 1 else np.array([], dtype=np.int64)
                ids = np.zeros(L, dtype=np.int32)
                for c in cuts:
                    ids[c:] += 1
                return ids
            q_doc = np.stack([runs(Lq) for _ in range(B)])
            kv_doc = q_doc if Lq == Lkv else np.stack([runs(Lkv) for _ in range(B)])
        else:
            q_doc = rng.integers(0, n_docs, size=(B, Lq)).astype(np.int32)
            kv_doc = q_doc if Lq == Lkv else rng.integers(0, n_docs, size=(B, Lkv)).astype(np.int32)
    slopes = rng.uniform(0.05, 0.8, size=Hq).astype(np.float32) if alibi else None
    q, k, v = _qkv(rng, B, Hq, Hkv, Lq, Lkv, D, dtype)
    return Workload(f"random_{seed}", dtype, B, Hq, Hkv, Lq, Lkv, D, q, k, v,
                    doc=doc, causal=causal, window=window, prefix_len=prefix_len,
                    softcap=softcap, alibi_slopes=slopes, q_doc=q_doc, kv_doc=kv_doc)


def grad_output(w: Workload, seed: int) -> np.ndarray:
    """A seeded output gradient dO for w: standard normal [B, Hq, Lq, D], in w's dtype
    (bf16 bit patterns or float32), from its own generator so that w's draws are unchanged."""
    rng = np.random.default_rng(10_000_000 + seed)
    return _normal(rng, (w.B, w.Hq, w.Lq, w.D), w.dtype)

"""Quantized form references: int8 Q/K, fp8 E4M3 V — TEST INFRASTRUCTURE.

The sage2 attention form (FlashRT-Structures PR #1, "LTX-2.5 attention forms")
runs Q.K^T on int8 and P.V on fp8 with bf16 output. The page gives INT8 Q/K with
fine-grained scales and FP8 per-channel V; the granularity used here is one
scale per (batch, head, 128-token block) for Q and K and one per (batch, head,
channel) for V, over all tokens. Rounding, which the page leaves open, is read
as: symmetric absmax scaling, scale and scaled values in float32 (correctly
rounded division), int8 codes by round-to-nearest-even clamped to +-127, E4M3
codes by round-to-nearest-even with saturation at +-448.

E4M3 is the OCP 8-bit floating point format E4M3 (the "FN" variant: exponent
bias 7, no infinities, S.1111.111 is NaN, largest finite 448, subnormals
m * 2^-9). Decoding and encoding are written from that definition.
"""
from __future__ import annotations

import numpy as np


def e4m3_decode(code: int) -> float:
    """Value of one E4M3 code (float; NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# The 127 non-negative finite values in code order (codes 0x00..0x7E); the
# order is increasing, so neighbouring values have neighbouring codes.
_POS_VALUES = np.array([e4m3_decode(c) for c in range(0x7F)], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes (uint8) for real values x: nearest, ties to even code, saturating.

    Magnitudes above 448 saturate to 448. -0.0 and negative values carry the
    sign bit.
    """
    x = np.asarray(x, dtype=np.float64)
    assert not np.isnan(x).any()
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")   # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def e4m3_decode_array(codes) -> np.ndarray:
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def quantize_int8_blocks(x_f32: np.ndarray, block: int = 128):
    """Int8 codes and float32 scales, one scale per (b, h, block of tokens).

    x_f32: float32 [B, H, L, D]. scale = amax / 127 (float32); code =
    rint(x / scale) clamped to +-127 (float32 division); amax == 0 gives
    scale 0 and codes 0. Returns (codes int8 [B,H,L,D], scales float32 [B,H,nb]).
    """
    x = np.asarray(x_f32, dtype=np.float32)
    B, H, L, D = x.shape
    nb = -(-L // block)
    codes = np.zeros(x.shape, dtype=np.int8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for i in range(nb):
        sl = x[:, :, i * block:(i + 1) * block, :]
        amax = np.abs(sl).max(axis=(2, 3)).astype(np.float32)
        scale = (amax / np.float32(127.0)).astype(np.float32)
        scales[:, :, i] = scale
        safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
        r = np.rint((sl / safe[:, :, None, None]).astype(np.float32))
        r = np.clip(r, -127, 127)
        r = np.where(scale[:, :, None, None] > 0, r, 0)
        codes[:, :, i * block:(i + 1) * block, :] = r.astype(np.int8)
    return codes, scales


def quantize_fp8_channels(x_f32: np.ndarray):
    """E4M3 codes and float32 scales, one scale per (b, h, channel) over all tokens.

    scale = amax / 448 (float32); code = E4M3(x / scale) with the quotient
    rounded to float32 first; amax == 0 gives scale 0 and codes 0.
    Returns (codes uint8 [B,H,L,D], scales float32 [B,H,D]).
    """
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.abs(x).max(axis=2).astype(np.float32)            # [B,H,D]
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / safe[:, :, None, :]).astype(np.float32)
    codes = e4m3_encode(y.astype(np.float64))
    codes = np.where(scale[:, :, None, :] > 0, codes, 0).astype(np.uint8)
    return codes, scale


def dequantize_int8(codes, scales, block: int = 128):
    c = np.asarray(codes, dtype=np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :c.shape[2]]
    return c * s[..., None]


def dequantize_fp8(codes, scales):
    return e4m3_decode_array(codes) * np.asarray(scales, dtype=np.float64)[:, :, None, :]


def attention_dequantized(q8, sq, k8, sk, v8, sv, rows, b, h, *, sm_scale=None, round_p=True):
    """Diagnostic: unmasked fp64 attention on dequantized inputs for some rows.

    P is rounded through E4M3 at a fixed x448 scale (P in [0, 1], relative to the
    final row maximum); the row sum uses the unrounded P. It bounds how much of the
    quantized form's error is the quantization itself. Pinned by two checks: without
    the P rounding it equals the attention oracle on the dequantized tensors, and a
    two-key case worked by hand puts 448 P on an E4M3 tie (tests/golden).
    """
    qh = dequantize_int8(q8[b:b + 1, h:h + 1], sq[b:b + 1, h:h + 1])[0, 0]
    kh = dequantize_int8(k8[b:b + 1, h:h + 1], sk[b:b + 1, h:h + 1])[0, 0]
    vh = dequantize_fp8(v8[b:b + 1, h:h + 1], sv[b:b + 1, h:h + 1])[0, 0]
    D = qh.shape[1]
    scale = 1.0 / np.sqrt(D) if not sm_scale else sm_scale
    s = qh[np.asarray(rows)] @ kh.T * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    pr = e4m3_decode_array(e4m3_encode(p * E4M3_MAX)) / E4M3_MAX if round_p else p
    return (pr @ vh) / l


# ---------------------------------------------------------------------------------------------
# Refinements of the form (FlashRT-Structures PR #1, "LTX-2.5 attention forms": the sage2 form
# takes Q/K scales per warp or per thread, and the fused prep of its FP4 sibling centres the
# inputs and applies a delta correction).
#
# Finer Q/K scales: quantize_int8_blocks with block=32 gives one scale per 32 tokens (one wave
# of 32 queries, or one 32-key sub-block of the kernel).
#
# K centering: K' = K - mu with mu[b, h, c] the mean of K over tokens. Softmax rows are
# invariant to adding a constant per row, and q_i . (k_j - mu) = q_i . k_j - q_i . mu, so the
# output is unchanged; only lse moves, by sm_scale * (q_i . mu), which the correction restores.
# Centering removes a common offset of the keys, so the int8 scale of a block follows the
# spread of the keys rather than their offset.
# ---------------------------------------------------------------------------------------------
def k_channel_mean(k_f32: np.ndarray) -> np.ndarray:
    """mu[b, h, c] = mean over tokens of K, as float32: the exactly rounded sum (math.fsum) divided
    by L in float64, then rounded to float32. L = 0 gives 0."""
    import math
    k = np.asarray(k_f32, dtype=np.float32)
    B, H, L, D = k.shape
    mu = np.zeros((B, H, D), dtype=np.float32)
    if L == 0:
        return mu
    for b in range(B):
        for h in range(H):
            for c in range(D):
                mu[b, h, c] = np.float32(math.fsum(k[b, h, :, c].astype(np.float64).tolist()) / L)
    return mu


def center_k(k_f32: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """K - mu per (b, h, channel), one float32 subtraction per element."""
    k = np.asarray(k_f32, dtype=np.float32)
    return (k - np.asarray(mu, dtype=np.float32)[:, :, None, :]).astype(np.float32)


def q_dot_mean(q_f32: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """delta[b, hq, i] = q_i . mu[b, hq // group] in float64 (the lse correction without sm_scale)."""
    q = np.asarray(q_f32, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    group = q.shape[1] // mu.shape[1]
    mq = np.repeat(mu, group, axis=1)                      # [B, Hq, D]
    return np.einsum("bhld,bhd->bhl", q, mq)

"""Gradients of the masked attention forward in float64 — TEST INFRASTRUCTURE.

FlexAttention guide, "Systems Mechanics", item 2 (automatic differentiation):
the backward of the fused forward gives dQ, dK and dV, differentiates the
score_mod (grad_score_mod), and lets gradients reach learnable score_mod
parameters such as ALiBi slopes. Here that derivative is written out by hand for
the fixed score_mod set of attention.py, per (batch, query head), with the score
matrix materialised row chunk by row chunk.

With r_ij = q_i . k_j (raw product), s = r * sm_scale, a = s - slope_h |i - j|
(ALiBi), f = C tanh(a / C) (soft-cap, else f = a), the masked softmax
P_ij = exp(f_ij - lse_i) (0 on masked pairs) and out_i = sum_j P_ij v_j:
  dv_j  = sum_i P_ij dout_i
  dP_ij = dout_i . v_j
  dF_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')      (softmax derivative)
  dA_ij = dF_ij (1 - (f_ij / C)^2)                (tanh' = 1 - tanh^2; dA = dF without soft-cap)
  dslope_h = sum_ij dA_ij * (-|i - j|)
  dR_ij = dA_ij * sm_scale
  dq_i  = sum_j dR_ij k_j,    dk_j = sum_i dR_ij q_i.
GQA: key/value head h // (Hq / Hkv) receives the sum over its query heads. A
query row with no allowed key has P = 0 and contributes nothing.

The row term sum_j P_ij dP_ij equals dout_i . out_i (the "delta" that a fused
backward computes from the stored forward output); the oracle uses the former.
"""
from __future__ import annotations

import numpy as np

from .attention import mask_mod, resolve_scale


def _slab(qh, kh, vh, doh, rows, b, hq, *, sm_scale, spec):
    """Gradient pieces of one (b, hq) slab for the given query rows.

    Returns (dq_rows, dk_part, dv_part, dslope_part).
    """
    Lkv = kh.shape[0]
    i = np.asarray(rows, np.int64).reshape(-1, 1)
    j = np.arange(Lkv, dtype=np.int64).reshape(1, -1)
    a = (qh[rows] @ kh.T) * sm_scale
    slope = None
    if spec.get("alibi_slopes") is not None:
        slope = float(np.float32(spec["alibi_slopes"][hq]))
        a = a - slope * np.abs(i - j).astype(np.float64)
    C = spec.get("softcap")
    f = float(C) * np.tanh(a / float(C)) if C is not None else a
    keep = mask_mod(rows, np.arange(Lkv),
                    q_doc_row=None if spec.get("q_doc") is None else spec["q_doc"][b],
                    kv_doc_row=None if spec.get("kv_doc") is None else spec["kv_doc"][b],
                    doc=spec.get("doc", False), causal=spec.get("causal", False),
                    window=spec.get("window"), prefix_len=spec.get("prefix_len"))
    fm = np.where(keep, f, -np.inf)
    m = fm.max(axis=1, keepdims=True)
    live = np.isfinite(m[:, 0])
    P = np.zeros_like(f)
    if live.any():
        e = np.exp(fm[live] - m[live])
        P[live] = e / e.sum(axis=1, keepdims=True)
    do = doh[rows]
    dP = do @ vh.T
    delta = (P * dP).sum(axis=1, keepdims=True)
    dF = P * (dP - delta)
    dA = dF * (1.0 - (f / float(C)) ** 2) if C is not None else dF
    dslope = float((dA * -np.abs(i - j).astype(np.float64)).sum()) if slope is not None else 0.0
    dR = dA * sm_scale
    return dR @ kh, dR.T @ qh[rows], P.T @ do, dslope


def attention_backward(q, k, v, dout, spec=None, *, chunk=512):
    """Gradients of attention.attention's output in float64.

    q: [B, Hq, Lq, D], k/v: [B, Hkv, Lkv, D], dout: [B, Hq, Lq, D] (widened to
    float64); spec as for attention.attention. Returns (dq, dk, dv, dslopes),
    dslopes float64 [Hq] (summed over batches) or None without ALiBi.
    """
    spec = dict(spec or {})
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    B, Hq, Lq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    sm_scale = resolve_scale(D, spec.get("sm_scale"))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dslopes = np.zeros(Hq) if spec.get("alibi_slopes") is not None else None
    for b in range(B):
        for hq in range(Hq):
            hk = hq // group
            for r0 in range(0, Lq, chunk):
                rows = np.arange(r0, min(Lq, r0 + chunk))
                gq, gk, gv, gs = _slab(q[b, hq], k[b, hk], v[b, hk], dout[b, hq], rows, b, hq,
                                       sm_scale=sm_scale, spec=spec)
                dq[b, hq, rows] = gq
                dk[b, hk] += gk
                dv[b, hk] += gv
                if dslopes is not None:
                    dslopes[hq] += gs
    return dq, dk, dv, dslopes

"""Dense fp64 masked attention: the definition the block-sparse kernel must reach.

Test infrastructure only (see oracle/__init__.py). Materialises the masked
score matrix for one (batch, query head) slab at a time, in query-row chunks.

Definition (FlexAttention guide, "The Core Design Principles"):
  s_ij   = q_i . k_j * sm_scale, sm_scale = 1/sqrt(d) unless given;
  s_ij   <- score_mod(s_ij, b, h, i, j): ALiBi bias then tanh soft-cap, the order
            of the guide's "Implementation" demo (bias added, then capped);
  keep   = mask_mod(b, h, i, j): AND of the enabled predicates;
  out_i  = sum_j softmax_j(s_i. restricted to keep) v_j;  lse_i = log sum_j exp(s_ij).

Readings where the pages are silent (each also in the design notes):
  * indices are absolute positions (no offset when Lq != Lkv);
  * window predicate is q - kv < W (strict); the demo's "<= 512" is W = 513;
  * prefix-LM is "kv < P or q >= kv" and already contains causal;
  * a query row with no allowed key gives out = 0 and lse = -inf;
  * lse is the natural logarithm;
  * GQA: query head h reads key/value head h // (Hq / Hkv).
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def mask_mod(i, j, *, q_doc_row=None, kv_doc_row=None, doc=False, causal=False,
             window=None, prefix_len=None):
    """Boolean mask for query positions i (column vector) and key positions j (row).

    FlexAttention guide: document packing (doc[q] == doc[kv], "Production
    Engineering" 1), causal q >= kv and sliding window (demo in
    "Implementation"), prefix-LM "kv < P or q >= kv" ("Production Engineering" 2).
    The enabled predicates are ANDed, as the demo ANDs causal and window.
    """
    i = np.asarray(i, dtype=np.int64).reshape(-1, 1)
    j = np.asarray(j, dtype=np.int64).reshape(1, -1)
    keep = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if doc:
        keep &= np.asarray(q_doc_row)[i] == np.asarray(kv_doc_row)[j]
    if causal:
        keep &= i >= j
    if window is not None:
        keep &= (i - j) < window
    if prefix_len is not None:
        keep &= (j < prefix_len) | (i >= j)
    return keep


def score_mod(s, i, j, *, alibi_slope=None, softcap=None):
    """Apply the score transforms to scaled scores s[i, j] (float64).

    ALiBi: s - slope * |i - j| (the demo's bias, slope of the query head).
    Soft-cap: C * tanh(s / C) (the guide's soft-cap formula, applied to the
    already scaled score, C = softcap).
    """
    s = np.array(s, dtype=np.float64, copy=True)
    if alibi_slope is not None:
        i = np.asarray(i, dtype=np.int64).reshape(-1, 1)
        j = np.asarray(j, dtype=np.int64).reshape(1, -1)
        s = s - float(alibi_slope) * np.abs(i - j).astype(np.float64)
    if softcap is not None:
        c = float(softcap)
        s = c * np.tanh(s / c)
    return s


def _rows(qh, kh, vh, rows, b, hq, *, sm_scale, spec):
    """Output and lse for the given query rows of one (b, hq) slab."""
    Lkv = kh.shape[0]
    j = np.arange(Lkv)
    s = (qh[rows] @ kh.T) * sm_scale
    slope = None if spec.get("alibi_slopes") is None else float(np.float32(spec["alibi_slopes"][hq]))
    s = score_mod(s, rows, j, alibi_slope=slope, softcap=spec.get("softcap"))
    keep = mask_mod(rows, j,
                    q_doc_row=None if spec.get("q_doc") is None else spec["q_doc"][b],
                    kv_doc_row=None if spec.get("kv_doc") is None else spec["kv_doc"][b],
                    doc=spec.get("doc", False), causal=spec.get("causal", False),
                    window=spec.get("window"), prefix_len=spec.get("prefix_len"))
    s[~keep] = -np.inf
    m = s.max(axis=1)
    out = np.zeros((len(rows), vh.shape[1]), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    live = np.isfinite(m)
    if live.any():
        p = np.exp(s[live] - m[live, None])
        l = p.sum(axis=1)
        out[live] = (p @ vh) / l[:, None]
        lse[live] = m[live] + np.log(l)
    return out, lse


def resolve_scale(D, sm_scale=None):
    """1/sqrt(D) unless a positive scale is given (guide's scaled score)."""
    if sm_scale is None or sm_scale <= 0:
        return 1.0 / math.sqrt(D)
    return float(sm_scale)


def attention(q, k, v, spec=None, *, chunk=1024):
    """Masked attention forward in float64.

    q: [B, Hq, Lq, D], k/v: [B, Hkv, Lkv, D] (float arrays, widened to float64).
    spec: dict with keys doc, causal, window, prefix_len, q_doc, kv_doc,
    alibi_slopes, softcap, sm_scale (all optional).
    Returns (out [B, Hq, Lq, D], lse [B, Hq, Lq]) in float64.
    """
    spec = dict(spec or {})
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Lq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    sm_scale = resolve_scale(D, spec.get("sm_scale"))
    out = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros((B, Hq, Lq), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = hq // group
            for r0 in range(0, Lq, chunk):
                rows = np.arange(r0, min(Lq, r0 + chunk))
                o, l = _rows(q[b, hq], k[b, hk], v[b, hk], rows, b, hq, sm_scale=sm_scale, spec=spec)
                out[b, hq, rows] = o
                lse[b, hq, rows] = l
    return out, lse


def attention_rows(q, k, v, spec, b, hq, rows):
    """Output and lse for selected query rows of one (b, hq); same definition."""
    spec = dict(spec or {})
    Hq, Hkv = q.shape[1], k.shape[1]
    hk = hq // (Hq // Hkv)
    qh = np.asarray(q[b, hq], dtype=np.float64)
    kh = np.asarray(k[b, hk], dtype=np.float64)
    vh = np.asarray(v[b, hk], dtype=np.float64)
    sm_scale = resolve_scale(q.shape[3], spec.get("sm_scale"))
    return _rows(qh, kh, vh, np.asarray(rows), b, hq, sm_scale=sm_scale, spec=spec)


def attention_by_groups(q, k, v, q_doc, *, sm_scale=None):
    """Attention under a document-equality mask only, evaluated group by group.

    Restates the document mask as block-diagonal attention: with packed
    contiguous ids and Lq == Lkv, each run of equal ids attends only within
    itself. Pinned against `attention` by the group-independence invariant.
    Returns (out, lse) like `attention`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Lq, D = q.shape
    group = Hq // k.shape[1]
    scale = resolve_scale(D, sm_scale)
    out = np.zeros(q.shape)
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        ids = np.asarray(q_doc[b])
        starts = np.flatnonzero(np.r_[True, ids[1:] != ids[:-1]])
        ends = np.r_[starts[1:], Lq]
        assert len(np.unique(ids[starts])) == len(starts), "ids must be contiguous runs"
        for hq in range(Hq):
            hk = hq // group
            for s0, e0 in zip(starts, ends):
                sc = q[b, hq, s0:e0] @ k[b, hk, s0:e0].T * scale
                m = sc.max(axis=1, keepdims=True)
                p = np.exp(sc - m)
                l = p.sum(axis=1, keepdims=True)
                out[b, hq, s0:e0] = (p @ v[b, hk, s0:e0]) / l
                lse[b, hq, s0:e0] = (m + np.log(l))[:, 0]
    return out, lse


def attention_by_documents_causal(q, k, v, q_doc, *, sm_scale=None):
    """Attention under document equality AND causality, evaluated document by document.

    Self-attention over packed documents (Lq == Lkv, one id array, each document a
    contiguous run of equal ids; guide, "Production Engineering" 1, with the
    demo's causal predicate): a query attends to the keys of its own run at or
    before its position, so each run is plain causal attention on its own slice.
    Pinned against `attention` with doc and causal on small packed cases.
    Returns (out, lse) like `attention`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Lq, D = q.shape
    assert k.shape[2] == Lq, "self-attention only"
    group = Hq // k.shape[1]
    scale = resolve_scale(D, sm_scale)
    out = np.zeros(q.shape)
    lse = np.zeros((B, Hq, Lq))
    for b in range(B):
        ids = np.asarray(q_doc[b])
        starts = np.flatnonzero(np.r_[True, ids[1:] != ids[:-1]])
        ends = np.r_[starts[1:], Lq]
        assert len(np.unique(ids[starts])) == len(starts), "ids must be contiguous runs"
        for s0, e0 in zip(starts, ends):
            n = e0 - s0
            upper = np.triu(np.ones((n, n), dtype=bool), 1)   # key after query: masked
            for hq in range(Hq):
                hk = hq // group
                sc = q[b, hq, s0:e0] @ k[b, hk, s0:e0].T * scale
                sc[upper] = -np.inf
                m = sc.max(axis=1, keepdims=True)               # the diagonal is always allowed
                p = np.exp(sc - m)
                l = p.sum(axis=1, keepdims=True)
                out[b, hq, s0:e0] = (p @ v[b, hk, s0:e0]) / l
                lse[b, hq, s0:e0] = (m + np.log(l))[:, 0]
    return out, lse


def attention_band(q, k, v, window, *, softcap=None, alibi_slopes=None, sm_scale=None, heads=None,
                   chunk=128):
    """Causal sliding-window attention (i >= j and i - j < window), evaluated on the band.

    Query rows [r0, r1) can only see keys [r0 - window + 1, r1), so only that band
    of the score matrix is materialised; score_mod (ALiBi, then soft-cap) and the
    two predicates are those of `attention`. Self-attention (Lq == Lkv).
    heads: optional list of (b, hq) to compute (others left 0). Pinned against
    `attention` with causal, window and the score transforms on small cases.
    Returns (out, lse) like `attention`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Lq, D = q.shape
    assert k.shape[2] == Lq, "self-attention only"
    group = Hq // k.shape[1]
    scale = resolve_scale(D, sm_scale)
    out = np.zeros(q.shape)
    lse = np.zeros((B, Hq, Lq))
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, hq in todo:
        hk = hq // group
        slope = None if alibi_slopes is None else float(np.float32(alibi_slopes[hq]))
        for r0 in range(0, Lq, chunk):
            r1 = min(Lq, r0 + chunk)
            c0 = max(0, r0 - window + 1)
            rows = np.arange(r0, r1)
            cols = np.arange(c0, r1)
            sc = q[b, hq, r0:r1] @ k[b, hk, c0:r1].T * scale
            sc = score_mod(sc, rows, cols, alibi_slope=slope, softcap=softcap)
            keep = mask_mod(rows, cols, causal=True, window=window)
            sc[~keep] = -np.inf
            m = sc.max(axis=1, keepdims=True)                   # j = i is always allowed
            p = np.exp(sc - m)
            l = p.sum(axis=1, keepdims=True)
            out[b, hq, r0:r1] = (p @ v[b, hk, c0:r1]) / l
            lse[b, hq, r0:r1] = (m + np.log(l))[:, 0]
    return out, lse

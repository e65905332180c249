"""Pure-Python loop attention for tiny inputs — TEST INFRASTRUCTURE.

An independent restatement of the definition with scalar loops and the math
module (no numpy arithmetic), used only to pin oracle/attention.py on tiny
shapes. Same definition and readings as attention.py (FlexAttention guide,
"The Core Design Principles", soft-cap formula in "The Problem", the
"Implementation" demo and the masks of "Production Engineering").
"""
from __future__ import annotations

import math


def allowed(b, i, j, spec):
    ok = True
    if spec.get("doc"):
        ok = ok and int(spec["q_doc"][b][i]) == int(spec["kv_doc"][b][j])
    if spec.get("causal"):
        ok = ok and i >= j
    if spec.get("window") is not None:
        ok = ok and (i - j) < spec["window"]
    if spec.get("prefix_len") is not None:
        ok = ok and (j < spec["prefix_len"] or i >= j)
    return ok


def attention(q, k, v, spec):
    """q: nested lists [B][Hq][Lq][D]; k, v: [B][Hkv][Lkv][D]. Returns (out, lse)."""
    B, Hq, Lq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Lkv = len(k[0]), len(k[0][0])
    scale = spec.get("sm_scale") or 1.0 / math.sqrt(D)
    out = [[[[0.0] * D for _ in range(Lq)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * Lq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(Lq):
                scores = []
                for j in range(Lkv):
                    if not allowed(b, i, j, spec):
                        continue
                    s = 0.0
                    for d in range(D):
                        s += float(q[b][h][i][d]) * float(k[b][hk][j][d])
                    s *= scale
                    if spec.get("alibi_slopes") is not None:
                        s += -float(spec["alibi_slopes"][h]) * abs(i - j)
                    if spec.get("softcap") is not None:
                        c = float(spec["softcap"])
                        s = c * math.tanh(s / c)
                    scores.append((j, s))
                if not scores:
                    lse[b][h][i] = -math.inf
                    continue
                m = max(s for _, s in scores)
                w = [(j, math.exp(s - m)) for j, s in scores]
                tot = sum(x for _, x in w)
                for d in range(D):
                    out[b][h][i][d] = sum(x * float(v[b][hk][j][d]) for j, x in w) / tot
                lse[b][h][i] = m + math.log(tot)
    return out, lse


def block_class(b, qb, kb, Lq, Lkv, BQ, BK, spec):
    """'full', 'partial' or 'empty' for one tile, by evaluating every in-range pair."""
    n_true = n_all = 0
    for i in range(qb * BQ, min(Lq, (qb + 1) * BQ)):
        for j in range(kb * BK, min(Lkv, (kb + 1) * BK)):
            n_all += 1
            n_true += 1 if allowed(b, i, j, spec) else 0
    if n_true == 0:
        return "empty"
    return "full" if n_true == n_all else "partial"

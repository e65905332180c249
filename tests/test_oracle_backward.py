"""Pins of the fp64 backward oracle (oracle/backward.py) and the transposed BlockMask.

- Library routine: torch autograd through CPU float64 scaled_dot_product_attention, for plain,
  causal, GQA, explicit-scale and document-masked attention; ALiBi enters SDPA as an additive
  float mask built from a slope tensor that requires grad, so autograd also gives dslope.
- Finite differences: central differences of the (separately pinned) forward oracle for the
  soft-cap, window and prefix-LM cases that SDPA cannot express, every score transform on.
- Invariants: sum_j dk_j = 0 without soft-cap (softmax rows of dF sum to zero); sum_j dv_j =
  sum of dout over live rows; fully masked rows give zero gradients.
- Transposed BlockMask: the transpose of the forward lists, and the causal closed form.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import backward as G
from oracle import blockmask as BM


def _rand(seed, B, Hq, Hkv, Lq, Lkv, D):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Hq, Lq, D)), r.standard_normal((B, Hkv, Lkv, D)),
            r.standard_normal((B, Hkv, Lkv, D)), r.standard_normal((B, Hq, Lq, D)))


def _sdpa_grads(q, k, v, do, *, causal=False, scale=None, bias_fn=None, slopes=None, keep=None):
    """Gradients from torch autograd through SDPA (float64, CPU).

    GQA by repeating kv heads (autograd sums the copies); bias_fn(slopes_t) gives an additive
    float mask [1, Hq, Lq, Lkv]; keep (bool [B, Lq, Lkv]) adds -inf on disallowed pairs."""
    t = lambda x: torch.tensor(np.ascontiguousarray(x), dtype=torch.float64, requires_grad=True)
    qt, kt, vt = t(q), t(k), t(v)
    Hq, Hkv = q.shape[1], k.shape[1]
    kr = kt.repeat_interleave(Hq // Hkv, dim=1)
    vr = vt.repeat_interleave(Hq // Hkv, dim=1)
    st = t(slopes) if slopes is not None else None
    mask = None
    if bias_fn is not None:
        mask = bias_fn(st)
    if keep is not None:
        km = torch.where(torch.from_numpy(keep)[:, None], 0.0, -torch.inf).to(torch.float64)
        mask = km if mask is None else mask + km
    out = torch.nn.functional.scaled_dot_product_attention(qt, kr, vr, attn_mask=mask, is_causal=causal,
                                                           scale=scale)
    out.backward(torch.from_numpy(do))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), (st.grad.numpy() if st is not None else None)


def _close(a, b, tol=1e-10):
    np.testing.assert_allclose(a, b, rtol=0, atol=tol * max(1.0, np.abs(b).max()))


@pytest.mark.parametrize("case", ["plain", "causal", "gqa", "scale"])
def test_matches_sdpa_autograd(case):
    if case == "gqa":
        q, k, v, do = _rand(1, 2, 8, 2, 29, 29, 16)
    else:
        q, k, v, do = _rand(2, 2, 3, 3, 33, 41 if case in ("plain", "scale") else 33, 16)
    spec, kw = {}, {}
    if case == "causal":
        spec["causal"], kw["causal"] = True, True
    if case == "scale":
        spec["sm_scale"], kw["scale"] = 0.37, 0.37
    got = G.attention_backward(q, k, v, do, spec)
    ref = _sdpa_grads(q, k, v, do, **kw)
    for g, r in zip(got[:3], ref[:3]):
        _close(g, r)
    assert got[3] is None


def test_alibi_and_doc_match_sdpa_autograd():
    B, H, L, D = 2, 4, 37, 8
    q, k, v, do = _rand(3, B, H, H, L, L, D)
    rng = np.random.default_rng(4)
    doc = np.sort(rng.integers(0, 4, size=(B, L)), axis=1).astype(np.int32)
    slopes = np.array([0.25, 0.5, 0.125, 0.0625], np.float32).astype(np.float64)
    spec = {"doc": True, "q_doc": doc, "kv_doc": doc, "alibi_slopes": slopes.astype(np.float32)}
    got = G.attention_backward(q, k, v, do, spec)
    dist = torch.from_numpy(np.abs(np.arange(L)[:, None] - np.arange(L)[None, :]).astype(np.float64))
    keep = doc[:, :, None] == doc[:, None, :]
    ref = _sdpa_grads(q, k, v, do, bias_fn=lambda s: (-s[:, None, None] * dist)[None], slopes=slopes, keep=keep)
    for g, r in zip(got, ref):
        _close(g, r)


def _loss(q, k, v, do, spec):
    out, _ = A.attention(q, k, v, spec)
    return float((out * do).sum())


@pytest.mark.parametrize("spec_name", ["softcap_alibi_window", "prefix_softcap_gqa"])
def test_finite_differences(spec_name):
    if spec_name == "softcap_alibi_window":
        q, k, v, do = _rand(5, 1, 2, 2, 13, 13, 4)
        spec = {"causal": True, "window": 5, "softcap": 1.5,
                "alibi_slopes": np.array([0.3, 0.7], np.float32)}
    else:
        q, k, v, do = _rand(6, 1, 4, 2, 11, 15, 4)
        spec = {"prefix_len": 6, "softcap": 2.0}
    q, k, v = q * 2.0, k * 2.0, v  # larger scores so that the soft-cap bends them
    dq, dk, dv, ds = G.attention_backward(q, k, v, do, spec)
    eps = 1e-6
    rng = np.random.default_rng(7)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, spec)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, spec)
            assert abs((fp - fm) / (2 * eps) - g[idx]) < 1e-7, (name, idx)
    if ds is not None:
        # The oracle reads slopes as float32: step each slope by a float32-representable amount.
        for h in range(len(spec["alibi_slopes"])):
            up = spec["alibi_slopes"].copy()
            dn = spec["alibi_slopes"].copy()
            up[h] += np.float32(1e-4)
            dn[h] -= np.float32(1e-4)
            fp = _loss(q, k, v, do, dict(spec, alibi_slopes=up))
            fm = _loss(q, k, v, do, dict(spec, alibi_slopes=dn))
            fd = (fp - fm) / (float(up[h]) - float(dn[h]))
            assert abs(fd - ds[h]) < 1e-6 * max(1.0, abs(ds[h])), (h, fd, ds[h])


def test_invariants():
    B, Hq, Hkv, L, D = 2, 4, 2, 40, 8
    q, k, v, do = _rand(8, B, Hq, Hkv, L, L, D)
    rng = np.random.default_rng(9)
    doc = np.sort(rng.integers(0, 5, size=(B, L)), axis=1).astype(np.int32)
    spec = {"doc": True, "q_doc": doc, "kv_doc": doc, "causal": True,
            "alibi_slopes": np.array([0.1, 0.2, 0.3, 0.4], np.float32)}
    dq, dk, dv, _ = G.attention_backward(q, k, v, do, spec)
    # Rows of dF sum to zero, so the key gradients of each (b, kv head) sum to zero.
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    # Rows of P sum to one: the value gradients add up to the summed output gradients.
    grp = Hq // Hkv
    for h in range(Hkv):
        np.testing.assert_allclose(dv[:, h].sum(axis=1), do[:, h * grp:(h + 1) * grp].sum(axis=(1, 2)), atol=1e-11)


def test_fully_masked_rows_have_zero_gradient():
    q, k, v, do = _rand(10, 1, 2, 2, 12, 12, 4)
    doc_q = np.array([[0] * 6 + [9] * 6], np.int32)
    doc_k = np.array([[0] * 12], np.int32)
    spec = {"doc": True, "q_doc": doc_q, "kv_doc": doc_k}
    dq, dk, dv, _ = G.attention_backward(q, k, v, do, spec)
    assert np.all(dq[:, :, 6:] == 0)
    ref = G.attention_backward(q[:, :, :6], k, v, do[:, :, :6], {})
    _close(dk, ref[1])
    _close(dv, ref[2])


@pytest.mark.parametrize("spec,L,BQ,BK", [
    ({"causal": True}, 1000, 128, 128),
    ({"causal": True, "window": 300}, 777, 128, 64),
    ({"prefix_len": 200}, 640, 128, 128),
])
def test_transposed_block_mask(spec, L, BQ, BK):
    fwd = BM.block_mask(spec, 1, L, L, BQ, BK)
    tr = BM.transposed_block_mask(spec, 1, L, L, BQ, BK)
    nqb, nkvb = fwd["kv_num_blocks"].shape[2], fwd["kv_indices"].shape[3]
    for kind, fk, tk in (("partial", "kv", "q"), ("full", "full_kv", "full_q")):
        pairs_f = {(qb, int(kb)) for qb in range(nqb) for kb in fwd[f"{fk}_indices"][0, 0, qb, :fwd[f"{fk}_num_blocks"][0, 0, qb]]}
        pairs_t = {(int(qb), kb) for kb in range(nkvb) for qb in tr[f"{tk}_indices"][0, 0, kb, :tr[f"{tk}_num_blocks"][0, 0, kb]]}
        assert pairs_f == pairs_t, kind
        for kb in range(nkvb):
            n = tr[f"{tk}_num_blocks"][0, 0, kb]
            lst = tr[f"{tk}_indices"][0, 0, kb]
            assert np.all(np.diff(lst[:n]) > 0) and np.all(lst[n:] == 0)
    if spec == {"causal": True} and BQ == BK:
        # Causal, square tiles: column kb has the diagonal tile partial and every later row full.
        n = -(-L // BQ)
        assert list(tr["q_num_blocks"][0, 0]) == [1] * n
        assert list(tr["full_q_num_blocks"][0, 0]) == [n - 1 - kb for kb in range(n)]


def test_group_independence():
    """With packed documents, the gradients of one document's tokens are those of the document
    alone (the full-size GPU checks compare slices cut at document boundaries)."""
    B, H, L, D = 1, 2, 60, 8
    q, k, v, do = _rand(11, B, H, H, L, L, D)
    doc = np.repeat(np.arange(4, dtype=np.int32), [10, 25, 5, 20])[None]
    spec = {"doc": True, "q_doc": doc, "kv_doc": doc, "causal": True}
    full = G.attention_backward(q, k, v, do, spec)
    s, e = 10, 40  # documents 1 and 2
    part = G.attention_backward(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], do[:, :, s:e],
                                dict(spec, q_doc=doc[:, s:e], kv_doc=doc[:, s:e]))
    for f, p in zip(full[:3], part[:3]):
        _close(f[:, :, s:e], p)

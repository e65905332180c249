"""Pins of the fp64 attention oracle against things other than itself.

Library routine (torch scaled_dot_product_attention, CPU float64), hand-worked
examples, invariants (group independence, masked keys contribute nothing,
softmax rows sum to one, soft-cap bound) and pure-Python brute force.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, B, Hq, Hkv, Lq, Lkv, D):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Hq, Lq, D)), r.standard_normal((B, Hkv, Lkv, D)),
            r.standard_normal((B, Hkv, Lkv, D)))


def _sdpa(q, k, v, **kw):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), **kw).numpy()


def test_hand_examples():
    ex = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["examples"]
    for e in ex:
        q = np.array(e["q"])[None, None]
        k = np.array(e["k"])[None, None]
        v = np.array(e["v"])[None, None]
        spec = {"softcap": e.get("softcap")}
        out, lse = A.attention(q, k, v, spec)
        np.testing.assert_allclose(out[0, 0], np.array(e["out"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], np.array(e["lse"]), rtol=0, atol=1e-14)


def test_plain_matches_sdpa():
    q, k, v = _rand(0, 2, 3, 3, 37, 53, 16)
    out, _ = A.attention(q, k, v, {})
    np.testing.assert_allclose(out, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_causal_matches_sdpa():
    q, k, v = _rand(1, 2, 2, 2, 45, 45, 8)
    out, _ = A.attention(q, k, v, {"causal": True})
    np.testing.assert_allclose(out, _sdpa(q, k, v, is_causal=True), rtol=0, atol=1e-12)


def test_gqa_matches_sdpa_with_repeated_heads():
    q, k, v = _rand(2, 1, 8, 2, 30, 30, 8)
    out, _ = A.attention(q, k, v, {})
    # Consecutive query heads share a KV head: repeat each KV head 4 times.
    ref = _sdpa(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_explicit_scale_matches_sdpa():
    q, k, v = _rand(3, 1, 2, 2, 20, 24, 8)
    out, _ = A.attention(q, k, v, {"sm_scale": 0.3})
    np.testing.assert_allclose(out, _sdpa(q, k, v, scale=0.3), rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one_and_reconstruct_output():
    q, k, v = _rand(4, 1, 2, 2, 33, 33, 8)
    spec = {"causal": True, "window": 9}
    out, lse = A.attention(q, k, v, spec)
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(8)
    i = np.arange(33)[:, None]
    j = np.arange(33)[None, :]
    keep = (i >= j) & (i - j < 9)
    w = np.where(keep, np.exp(s - lse[..., None]), 0.0)
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.einsum("bhij,bhjd->bhid", w, v), out, rtol=0, atol=1e-12)


def _doc_runs(seed, L, n):
    r = np.random.default_rng(seed)
    cuts = np.sort(r.choice(np.arange(1, L), n - 1, replace=False))
    ids = np.zeros(L, np.int32)
    for c in cuts:
        ids[c:] += 1
    return ids


def test_doc_mask_equals_independent_groups_sdpa():
    q, k, v = _rand(5, 2, 2, 2, 90, 90, 16)
    docs = np.stack([_doc_runs(6, 90, 7), _doc_runs(7, 90, 4)])
    out, lse = A.attention(q, k, v, {"doc": True, "q_doc": docs, "kv_doc": docs})
    for b in range(2):
        ids = docs[b]
        for g in np.unique(ids):
            sl = np.flatnonzero(ids == g)
            ref = _sdpa(q[b:b + 1, :, sl], k[b:b + 1, :, sl], v[b:b + 1, :, sl])
            np.testing.assert_allclose(out[b:b + 1, :, sl], ref, rtol=0, atol=1e-12)
    out2, lse2 = A.attention_by_groups(q, k, v, docs)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def test_single_group_equals_dense():
    q, k, v = _rand(8, 1, 2, 2, 40, 40, 8)
    docs = np.zeros((1, 40), np.int32)
    out, lse = A.attention(q, k, v, {"doc": True, "q_doc": docs, "kv_doc": docs})
    out0, lse0 = A.attention(q, k, v, {})
    np.testing.assert_array_equal(out, out0)
    np.testing.assert_array_equal(lse, lse0)


@pytest.mark.parametrize("spec_kind", ["doc", "causal_window", "prefix"])
def test_masked_keys_contribute_exactly_zero(spec_kind):
    B, H, L, D = 1, 2, 50, 8
    q, k, v = _rand(9, B, H, H, L, L, D)
    docs = _doc_runs(10, L, 5)[None]
    spec = {"doc": {"doc": True, "q_doc": docs, "kv_doc": docs},
            "causal_window": {"causal": True, "window": 7},
            "prefix": {"prefix_len": 6}}[spec_kind]
    out, lse = A.attention(q, k, v, spec)
    keep = A.mask_mod(np.arange(L), np.arange(L), q_doc_row=docs[0], kv_doc_row=docs[0],
                      doc=spec.get("doc", False), causal=spec.get("causal", False),
                      window=spec.get("window"), prefix_len=spec.get("prefix_len"))
    # Rewrite K and V where a key is masked for a chosen query row: the row's
    # output and lse stay bit-identical (same code path before and after).
    for i in range(0, L, 7):
        k2, v2 = k.copy(), v.copy()
        bad = ~keep[i]
        k2[:, :, bad] = 1e3
        v2[:, :, bad] = -1e3
        o1, l1 = A.attention_rows(q, k, v, spec, 0, 1, [i])
        o2, l2 = A.attention_rows(q, k2, v2, spec, 0, 1, [i])
        assert np.array_equal(o2, o1) and np.array_equal(l2, l1)
        np.testing.assert_allclose(o1[0], out[0, 1, i], rtol=0, atol=1e-12)


def test_softcap_bound_and_limit():
    q, k, v = _rand(11, 1, 2, 2, 30, 30, 8)
    q *= 20
    s = A.score_mod(np.einsum("id,jd->ij", q[0, 0], k[0, 0]), np.arange(30), np.arange(30), softcap=5.0)
    assert np.abs(s).max() <= 5.0
    o_big, l_big = A.attention(q, k, v, {"softcap": 1e12})
    o_none, l_none = A.attention(q, k, v, {})
    np.testing.assert_allclose(o_big, o_none, rtol=0, atol=1e-9)
    np.testing.assert_allclose(l_big, l_none, rtol=0, atol=1e-9)


def test_alibi_zero_slopes_equal_none():
    q, k, v = _rand(12, 1, 3, 3, 25, 25, 8)
    o1, l1 = A.attention(q, k, v, {"alibi_slopes": np.zeros(3, np.float32), "causal": True})
    o0, l0 = A.attention(q, k, v, {"causal": True})
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(l1, l0)


def test_prefix_lm_limits():
    q, k, v = _rand(13, 1, 2, 2, 33, 33, 8)
    o, _ = A.attention(q, k, v, {"prefix_len": 0})
    np.testing.assert_allclose(o, _sdpa(q, k, v, is_causal=True), rtol=0, atol=1e-12)
    o, _ = A.attention(q, k, v, {"prefix_len": 33})
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_wide_window_equals_causal():
    q, k, v = _rand(14, 1, 2, 2, 33, 33, 8)
    o, _ = A.attention(q, k, v, {"causal": True, "window": 33})
    np.testing.assert_allclose(o, _sdpa(q, k, v, is_causal=True), rtol=0, atol=1e-12)


def test_fully_masked_rows():
    q, k, v = _rand(15, 1, 1, 1, 6, 6, 4)
    qd = np.array([[0, 0, 1, 2, 2, 9]], np.int32)
    kd = np.array([[0, 0, 1, 2, 2, 3]], np.int32)
    out, lse = A.attention(q, k, v, {"doc": True, "q_doc": qd, "kv_doc": kd})
    assert np.all(out[0, 0, 5] == 0) and lse[0, 0, 5] == -np.inf
    assert np.isfinite(lse[0, 0, :5]).all()


def _nested(x):
    return x.tolist()


SPECS = [
    {},
    {"causal": True},
    {"doc": True},
    {"doc": True, "causal": True},
    {"causal": True, "window": 5},
    {"window": 4},
    {"prefix_len": 7},
    {"doc": True, "prefix_len": 3},
    {"doc": True, "causal": True, "window": 6},
    {"prefix_len": 5, "window": 9},
]


@pytest.mark.parametrize("si", range(len(SPECS)))
@pytest.mark.parametrize("score", ["none", "alibi", "softcap", "both"])
def test_brute_force_all_combinations(si, score):
    B, Hq, Hkv, Lq, Lkv, D = 2, 4, 2, 19, 23, 5
    q, k, v = _rand(100 + si, B, Hq, Hkv, Lq, Lkv, D)
    r = np.random.default_rng(200 + si)
    spec = dict(SPECS[si])
    if spec.get("doc"):
        spec["q_doc"] = r.integers(0, 3, (B, Lq)).astype(np.int32)
        spec["kv_doc"] = r.integers(0, 3, (B, Lkv)).astype(np.int32)
    if score in ("alibi", "both"):
        spec["alibi_slopes"] = r.uniform(0.1, 0.8, Hq).astype(np.float32)
    if score in ("softcap", "both"):
        spec["softcap"] = 2.5
        q = q * 3
    out, lse = A.attention(q, k, v, spec)
    bo, bl = brute.attention(_nested(q), _nested(k), _nested(v), spec)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    bl = np.array(bl)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], np.uint16)
    vals = A.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0
    assert np.signbit(vals[3]) and vals[3] == 0.0
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127
    assert vals[5] == 2.0 ** -133
    assert vals[6] == 3.140625


def test_documents_causal_restatement():
    """attention_by_documents_causal: every document equals causal SDPA on its own slice (library
    routine), and the whole equals the definition with doc AND causal, GQA included."""
    q, k, v = _rand(21, 2, 4, 2, 150, 150, 16)
    docs = np.stack([_doc_runs(22, 150, 9), _doc_runs(23, 150, 3)])
    out, lse = A.attention_by_documents_causal(q, k, v, docs)
    for b in range(2):
        for g in np.unique(docs[b]):
            sl = np.flatnonzero(docs[b] == g)
            kk = np.repeat(k[b:b + 1, :, sl], 2, axis=1)
            vv = np.repeat(v[b:b + 1, :, sl], 2, axis=1)
            ref = _sdpa(q[b:b + 1, :, sl], kk, vv, is_causal=True)
            np.testing.assert_allclose(out[b:b + 1, :, sl], ref, rtol=0, atol=1e-12)
    o_def, l_def = A.attention(q, k, v, {"doc": True, "causal": True, "q_doc": docs, "kv_doc": docs})
    np.testing.assert_allclose(out, o_def, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_def, rtol=0, atol=1e-12)
    # One document is plain causal attention.
    one = np.zeros((2, 150), np.int32)
    o1, _ = A.attention_by_documents_causal(q, k, v, one)
    ref = _sdpa(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), is_causal=True)
    np.testing.assert_allclose(o1, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window,score", [(1, None), (7, None), (40, "softcap"), (64, "alibi_softcap"), (300, None)])
def test_band_restatement(window, score):
    """attention_band equals the definition with causal AND window (and the score transforms);
    window 1 keeps only the diagonal (out_i = v_i, lse_i = s_ii); a window wider than the
    sequence is causal SDPA (library routine)."""
    q, k, v = _rand(30 + window, 2, 4, 2, 260, 260, 16)
    kw, spec = {}, {"causal": True, "window": window}
    if score:
        kw["softcap"] = spec["softcap"] = 1.5
    if score == "alibi_softcap":
        kw["alibi_slopes"] = spec["alibi_slopes"] = np.linspace(0.1, 0.8, 4).astype(np.float32)
    out, lse = A.attention_band(q, k, v, window, chunk=64, **kw)
    o_def, l_def = A.attention(q, k, v, spec)
    np.testing.assert_allclose(out, o_def, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_def, rtol=0, atol=1e-12)
    if window == 1:
        np.testing.assert_allclose(out, np.repeat(v, 2, axis=1), rtol=0, atol=1e-15)
        s_ii = np.einsum("bhld,bhld->bhl", q, np.repeat(k, 2, axis=1)) / 4.0
        np.testing.assert_allclose(lse, s_ii, rtol=0, atol=1e-12)
    if window == 300:
        ref = _sdpa(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), is_causal=True)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # Selected heads only.
    o_h, _ = A.attention_band(q, k, v, window, heads=[(1, 3)], chunk=64, **kw)
    np.testing.assert_array_equal(o_h[1, 3], out[1, 3])
    assert not o_h[0].any()

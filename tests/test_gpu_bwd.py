"""GPU: backward parity (dQ, dK, dV, ALiBi-slope gradient) with the fp64 backward oracle.

The GPU forward provides out and lse (the backward's inputs); the oracle recomputes everything
from q, k, v and dout. Small seeded cases cover every mask and score combination with GQA,
ragged tails and Lq != Lkv; then a NULL BlockMask, GQA ratios, fully masked rows, empty inputs,
strided views and an explicit scale. Full-size workloads are compared on slices whose rows
see only keys inside the slice (whole documents or groups; for the sliding window, rows and
keys at least one window from the slice's edges), on sampled dQ rows (row-local), and through
two invariants that hold at any size: sum_j dK_j = 0 without soft-cap and sum_j dV_j =
sum_i dO_i over rows with an allowed key.

Tolerance (bf16 gradients; P and dA are rounded to bf16 before their products, as in the
forward): max |G - ref| <= 2e-2 * max(1, max |ref|) and cosine >= 0.9999 per gradient; the
slope gradient within 2e-2 of max(1, max |ref|).
"""
import numpy as np
import pytest

from oracle import backward as ref_bwd
from oracle import blockmask as ref_bm
from tests._util import cosine, to_device
from tests.test_gpu_fwd import CASES, SCORES, mask_kind, score_kind, spec_of
from workloads import grad_output, make_workload, random_case

pytestmark = pytest.mark.gpu

TOL_ABS = 2e-2
TOL_COS = 0.9999


def _fa():
    import block_sparse_masked_blockmask_amd as fa
    return fa


def _tensors(w, dev, dout):
    import torch
    q, k, v = (to_device(x, w.dtype, dev) for x in (w.q, w.k, w.v))
    do = to_device(dout, w.dtype, dev)
    qd = kd = sl = None
    if w.doc:
        qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
        kd = torch.from_numpy(np.ascontiguousarray(w.kv_doc)).to(dev)
    if w.alibi_slopes is not None:
        sl = torch.from_numpy(w.alibi_slopes).to(dev)
    return q, k, v, do, qd, kd, sl


def run_fwd_bwd(w, dout, use_bm=True, sm_scale=0.0, views=None):
    """GPU forward then backward; returns (dq, dk, dv, dslopes, bm) as numpy float64 (bm on device)."""
    import torch
    fa = _fa()
    dev = torch.device("cuda", 0)
    q, k, v, do, qd, kd, sl = _tensors(w, dev, dout)
    if views is not None:
        q, k, v, do = views(q, k, v, do)
    mk, sk = mask_kind(w), score_kind(w)
    kw = dict(window=w.window or 0, prefix_len=w.prefix_len or 0, softcap=w.softcap or 0.0, alibi_slopes=sl,
              q_doc=qd, kv_doc=kd, sm_scale=sm_scale)
    bm = None
    if use_bm:
        bm = fa.flexattn_block_mask_build(mk, w.B, w.Lq, w.Lkv, 128, 128, q_doc=qd, kv_doc=kd,
                                          window=w.window or 0, prefix_len=w.prefix_len or 0, device=dev)
    out, lse = fa.flexattn_fwd(q, k, v, bm, mk, sk, **kw)
    dq, dk, dv, ds = fa.flexattn_bwd(q, k, v, out, do, lse, bm, None, mk, sk, slope_grad=w.alibi_slopes is not None,
                                     **kw)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return f(dq), f(dk), f(dv), (ds.cpu().numpy().astype(np.float64) if ds is not None else None), bm


def _f32(x, dtype):
    from workloads import bf16_bits_to_f32
    return bf16_bits_to_f32(x) if dtype == "bf16" else x


def check_grad(got, ref, what):
    scale = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= TOL_ABS * scale, f"{what}: max err {err:.3e} > {TOL_ABS * scale:.3e}"
    if ref.size and np.abs(ref).max() > 0:
        c = cosine(got, ref)
        assert c >= TOL_COS, f"{what}: cosine {c:.7f}"
    return err / scale


def check_all(got, ref, what):
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        check_grad(g, r, f"{what} {name}")
    if ref[3] is not None:
        scale = max(1.0, float(np.abs(ref[3]).max()))
        err = float(np.abs(got[3] - ref[3]).max())
        assert err <= TOL_ABS * scale, f"{what} dslopes: {got[3]} vs {ref[3]}"


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("si", range(len(SCORES)))
def test_small_cases(ci, si):
    kw = dict(CASES[ci])
    kw.update(SCORES[si])
    Lq, Lkv = (333, 333) if kw.get("doc") else (333, 401)
    w = random_case(10 * ci + si, dtype="bf16", B=2, Hq=4, Hkv=2, Lq=Lq, Lkv=Lkv, **kw)
    dout = grad_output(w, 10 * ci + si)
    got = run_fwd_bwd(w, dout)
    qf, kf, vf = w.qkv_f32()
    ref = ref_bwd.attention_backward(qf, kf, vf, _f32(dout, "bf16"), spec_of(w))
    check_all(got, ref, f"case {ci}/{si}")
    if ci == 3 and si == 0:
        # The transposed BlockMask built inside the call equals the oracle's column view.
        fa = _fa()
        bmt = fa.flexattn_block_mask_transpose(got[4])
        exp = ref_bm.transposed_block_mask(spec_of(w), w.B, w.Lq, w.Lkv, 128, 128)
        for key in exp:
            assert np.array_equal(getattr(bmt, key).cpu().numpy(), exp[key]), key


@pytest.mark.parametrize("case", ["causal_window", "doc_unsorted", "prefix"])
def test_transpose_bit_exact(case):
    """The device transpose against the oracle's column view, with 64-wide tiles too."""
    import torch
    fa = _fa()
    dev = torch.device("cuda", 0)
    kw = {"causal_window": dict(causal=True, window=300), "doc_unsorted": dict(doc=True, n_docs=5, doc_sorted=False),
          "prefix": dict(prefix_len=200)}[case]
    w = random_case(77, dtype="bf16", B=2, Hq=2, Lq=900, Lkv=900 if case == "doc_unsorted" else 1000, **kw)
    qd = kd = None
    if w.doc:
        qd = torch.from_numpy(w.q_doc).to(dev)
        kd = torch.from_numpy(w.kv_doc).to(dev)
    for qb, kb in ((128, 128), (128, 64), (64, 128)):
        bm = fa.flexattn_block_mask_build(mask_kind(w), w.B, w.Lq, w.Lkv, qb, kb, q_doc=qd, kv_doc=kd,
                                          window=w.window or 0, prefix_len=w.prefix_len or 0, device=dev)
        bmt = fa.flexattn_block_mask_transpose(bm)
        torch.cuda.synchronize()
        exp = ref_bm.transposed_block_mask(spec_of(w), w.B, w.Lq, w.Lkv, qb, kb)
        for key in exp:
            assert np.array_equal(getattr(bmt, key).cpu().numpy(), exp[key]), (case, qb, kb, key)


def test_null_block_mask_and_gqa_ratios():
    for group in (1, 2, 4, 8):
        w = random_case(600 + group, dtype="bf16", B=1, Hq=8, Hkv=8 // group, Lq=200, Lkv=300)
        dout = grad_output(w, 600 + group)
        got = run_fwd_bwd(w, dout, use_bm=False)
        qf, kf, vf = w.qkv_f32()
        check_all(got, ref_bwd.attention_backward(qf, kf, vf, _f32(dout, "bf16"), {}), f"null bm group {group}")


def test_fully_masked_rows():
    w = random_case(610, dtype="bf16", B=1, Hq=2, Lq=300, Lkv=300, doc=True, n_docs=4, doc_sorted=False, alibi=True)
    w.q_doc = w.q_doc.copy()
    w.q_doc[0, 5] = 99
    w.q_doc[0, 256:] = 77
    dout = grad_output(w, 610)
    got = run_fwd_bwd(w, dout)
    qf, kf, vf = w.qkv_f32()
    ref = ref_bwd.attention_backward(qf, kf, vf, _f32(dout, "bf16"), spec_of(w))
    assert np.all(got[0][0, :, 5] == 0) and np.all(got[0][0, :, 256:] == 0)
    check_all(got, ref, "masked rows")


@pytest.mark.parametrize("Lq,Lkv", [(0, 100), (100, 0), (0, 0)])
def test_empty_inputs(Lq, Lkv):
    import torch
    w = random_case(620, dtype="bf16", B=1, Hq=2, Lq=max(Lq, 1), Lkv=max(Lkv, 1), alibi=True)
    w.q, w.k, w.v = w.q[:, :, :Lq], w.k[:, :, :Lkv], w.v[:, :, :Lkv]
    w.Lq, w.Lkv = Lq, Lkv
    dout = grad_output(w, 620)
    dq, dk, dv, ds, _ = run_fwd_bwd(w, dout, use_bm=False)
    assert dq.shape == (1, 2, Lq, 128) and dk.shape == (1, 2, Lkv, 128)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0) and np.all(ds == 0)


def test_strided_views_and_scale():
    # [B, L, H, D] storage viewed as [B, H, L, D], and an explicit sm_scale.
    w = random_case(630, dtype="bf16", B=2, Hq=4, Hkv=2, Lq=257, Lkv=311, causal=True, alibi=True, softcap=25.0)
    dout = grad_output(w, 630)

    def views(q, k, v, do):
        return tuple(x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v, do))
    got = run_fwd_bwd(w, dout, sm_scale=0.05, views=views)
    qf, kf, vf = w.qkv_f32()
    ref = ref_bwd.attention_backward(qf, kf, vf, _f32(dout, "bf16"), dict(spec_of(w), sm_scale=0.05))
    check_all(got, ref, "strided+scale")


def _slice(w, dout, s, e, hkv=1):
    """Copy of w restricted to batch 0, the first hkv kv heads (with their query heads) and
    tokens [s, e) (self-attention workloads)."""
    import copy
    u = copy.copy(w)
    hq = hkv * (w.Hq // w.Hkv)
    u.q, u.k, u.v = w.q[:1, :hq, s:e], w.k[:1, :hkv, s:e], w.v[:1, :hkv, s:e]
    u.B, u.Hq, u.Hkv = 1, hq, hkv
    u.Lq = u.Lkv = e - s
    if w.doc:
        u.q_doc = np.ascontiguousarray(w.q_doc[:1, s:e])
        u.kv_doc = np.ascontiguousarray(w.kv_doc[:1, s:e])
    if w.alibi_slopes is not None:
        u.alibi_slopes = w.alibi_slopes[:hq]
    return u, dout[:1, :hq, s:e]


def _dq_rows(w, dout, b, hq, rows):
    """Oracle dQ for some rows of one (b, hq): row-local, needs only those rows' scores."""
    qf, kf, vf = w.qkv_f32()
    hk = hq // (w.Hq // w.Hkv)
    sm = 1.0 / np.sqrt(w.D)
    gq, _, _, _ = ref_bwd._slab(qf[b, hq].astype(np.float64), kf[b, hk].astype(np.float64),
                                vf[b, hk].astype(np.float64), _f32(dout, w.dtype)[b, hq].astype(np.float64),
                                np.asarray(rows), b, hq, sm_scale=sm, spec=spec_of(w))
    return gq


@pytest.mark.parametrize("name", ["grouped_variate_4096g_bf16", "doc_causal_b4h16t8192_bf16",
                                  "swa1024_gqa32x8_softcap50_t16384_bf16", "dense_b1h32s24576_bf16"])
def test_workloads_full_size(name):
    w = make_workload(name)
    dout = grad_output(w, 900)
    dq, dk, dv, ds, _ = run_fwd_bwd(w, dout)
    rng = np.random.default_rng(901)
    qf, kf, vf = w.qkv_f32()
    do64 = _f32(dout, w.dtype).astype(np.float64)
    # Sampled dQ rows (first, last, random) of a few heads.
    for b, hq in ((0, 0), (w.B - 1, w.Hq - 1), (0, w.Hq // 2)):
        rows = np.unique(np.r_[0, w.Lq - 1, rng.integers(0, w.Lq, 40)])
        check_grad(dq[b, hq, rows], _dq_rows(w, dout, b, hq, rows), f"{name} dq rows b{b} h{hq}")
    # Slices whose rows see only keys inside them (batch 0, the first kv head and its query heads).
    hq = w.Hq // w.Hkv
    if w.doc:
        ids = w.q_doc[0]
        starts = np.flatnonzero(np.r_[True, ids[1:] != ids[:-1]])
        s = int(starts[len(starts) // 2])
        e = int(starts[min(len(starts) - 1, np.searchsorted(starts, s + 600))])
        u, du = _slice(w, dout, s, e)
        uq, uk, uv = u.qkv_f32()
        ref = ref_bwd.attention_backward(uq, uk, uv, _f32(du, w.dtype), spec_of(u))
        check_grad(dq[:1, :hq, s:e], ref[0], f"{name} slice dq")
        check_grad(dk[:1, :1, s:e], ref[1], f"{name} slice dk")
        check_grad(dv[:1, :1, s:e], ref[2], f"{name} slice dv")
    elif w.window is not None:
        W = w.window
        s, e = w.Lq // 2, w.Lq // 2 + 3 * W
        u, du = _slice(w, dout, s, e)
        uq, uk, uv = u.qkv_f32()
        ref = ref_bwd.attention_backward(uq, uk, uv, _f32(du, w.dtype), spec_of(u))
        check_grad(dq[:1, :hq, s + W:e], ref[0][:, :, W:], f"{name} slice dq")
        check_grad(dk[:1, :1, s + W:e - W], ref[1][:, :, W:2 * W], f"{name} slice dk")
        check_grad(dv[:1, :1, s + W:e - W], ref[2][:, :, W:2 * W], f"{name} slice dv")
    # Invariants at full size (float64 sums of the bf16 gradients), per (b, head, channel):
    # sum_j dK_j = 0 (no soft-cap) and sum_j dV_j = sum over the group's rows of dO (every row of
    # these workloads has an allowed key). Tolerance: 2e-2 of the root sum of squares, several
    # times the bf16 rounding of the summed gradients.
    if not w.softcap:
        err = np.abs(dk.sum(axis=2))
        assert np.all(err <= 2e-2 * np.sqrt((dk ** 2).sum(axis=2)) + 1e-3), f"{name}: sum_j dK_j"
    for h in range(w.Hkv):
        exp = do64[:, h * hq:(h + 1) * hq].sum(axis=(1, 2))
        err = np.abs(dv[:, h].sum(axis=1) - exp)
        assert np.all(err <= 2e-2 * np.sqrt((dv[:, h] ** 2).sum(axis=1)) + 1e-3), f"{name}: sum_j dV_j"


def test_backward_with_schedule_bit_identical():
    """A BlockMask and transpose carrying the cost-ordered schedules change only when the dq
    and dk/dv passes' work items run: dq, dk, dv and the slope gradient are bit-identical to
    the plain ones'."""
    import torch
    import block_sparse_masked_blockmask_amd as fa
    from tests._util import to_device
    from workloads import grad_output, random_case
    dev = torch.device("cuda", 0)
    w = random_case(4700, dtype="bf16", B=2, Hq=4, Hkv=2, Lq=1500, Lkv=1500, doc=True, causal=True, alibi=True)
    q, k, v = (to_device(x, "bf16", dev) for x in (w.q, w.k, w.v))
    do = to_device(grad_output(w, 4700), "bf16", dev)
    qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
    sl = torch.from_numpy(w.alibi_slopes).to(dev)
    mk, sk = fa.FA_MASK_DOC | fa.FA_MASK_CAUSAL, fa.FA_SCORE_ALIBI
    res = []
    for order in (False, True):
        bm = fa.flexattn_block_mask_build(mk, w.B, w.Lq, w.Lkv, 128, 128, q_doc=qd, kv_doc=qd, device=dev,
                                          row_order=order)
        bmt = fa.flexattn_block_mask_transpose(bm, col_order=order)
        if order:
            # The column schedule: kv blocks by decreasing 4 * full + 5 * partial, ties by kv block.
            fullc = bmt.full_q_num_blocks.cpu().numpy().astype(np.int64)
            partc = bmt.q_num_blocks.cpu().numpy().astype(np.int64)
            got = bmt.col_order.cpu().numpy()
            for bb in range(got.shape[0]):
                cost = 4 * fullc[bb, 0] + 5 * partc[bb, 0]
                want = sorted(range(got.shape[-1]), key=lambda kb: (-cost[kb], kb))
                assert list(got[bb, 0]) == want
        out, lse = fa.flexattn_fwd(q, k, v, bm, mk, sk, alibi_slopes=sl, q_doc=qd, kv_doc=qd)
        dq, dk, dv, ds = fa.flexattn_bwd(q, k, v, out, do, lse, bm, bmt, mk, sk, alibi_slopes=sl, q_doc=qd, kv_doc=qd,
                                         slope_grad=True)
        torch.cuda.synchronize()
        res.append([t.float().cpu() for t in (out, lse, dq, dk, dv, ds)])
    for a, b in zip(*res):
        assert torch.equal(a, b)

"""GPU: forward parity with the fp64 oracle, element by element.

Small seeded cases cover every mask and score combination, GQA, Lq != Lkv, ragged tails,
both kv block sizes, fully masked rows, empty BlockMask rows and NULL BlockMask; the
workloads run at full size in the bench's launch configuration and are compared on
sampled query rows (the oracle computes those rows one by one) and, for the grouped
workload, on the whole output through the per-group restatement of the oracle.
"""
import numpy as np
import pytest

from oracle import attention as ref_attn
from oracle import blockmask as ref_bm
from tests._util import check_close, cosine, to_device
from workloads import make_workload, random_case

pytestmark = pytest.mark.gpu


def _fa():
    import block_sparse_masked_blockmask_amd as fa
    return fa


def mask_kind(w):
    fa = _fa()
    m = 0
    m |= fa.FA_MASK_DOC if w.doc else 0
    m |= fa.FA_MASK_CAUSAL if w.causal else 0
    m |= fa.FA_MASK_WINDOW if w.window is not None else 0
    m |= fa.FA_MASK_PREFIX_LM if w.prefix_len is not None else 0
    return m


def score_kind(w):
    fa = _fa()
    return (fa.FA_SCORE_ALIBI if w.alibi_slopes is not None else 0) | (fa.FA_SCORE_SOFTCAP if w.softcap else 0)


def spec_of(w):
    return dict(doc=w.doc, causal=w.causal, window=w.window, prefix_len=w.prefix_len, q_doc=w.q_doc,
                kv_doc=w.kv_doc, alibi_slopes=w.alibi_slopes, softcap=w.softcap)


def run_gpu(w, kv_block=128, use_bm=True, lse=True, q_block=128):
    """Build the BlockMask and run the forward on the GPU; returns (out, lse, bm, tensors)."""
    import torch
    fa = _fa()
    dev = torch.device("cuda", 0)
    q, k, v = (to_device(x, w.dtype, dev) for x in (w.q, w.k, w.v))
    qd = kd = sl = None
    if w.doc:
        qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
        kd = torch.from_numpy(np.ascontiguousarray(w.kv_doc)).to(dev)
    if w.alibi_slopes is not None:
        sl = torch.from_numpy(w.alibi_slopes).to(dev)
    mk, sk = mask_kind(w), score_kind(w)
    bm = None
    if use_bm:
        bm = fa.flexattn_block_mask_build(mk, w.B, w.Lq, w.Lkv, q_block, kv_block, q_doc=qd, kv_doc=kd,
                                          window=w.window or 0, prefix_len=w.prefix_len or 0, device=dev)
    out, l = fa.flexattn_fwd(q, k, v, bm, mk, sk, window=w.window or 0, prefix_len=w.prefix_len or 0,
                             softcap=w.softcap or 0.0, alibi_slopes=sl, q_doc=qd, kv_doc=kd, return_lse=lse)
    torch.cuda.synchronize()
    return out, l, bm


# The BlockMask block sizes bench.py uses per dtype (q_block, kv_block).
BENCH_BLOCKS = {"bf16": (128, 64), "f32": (128, 128)}

CASES = [
    dict(),
    dict(causal=True),
    dict(doc=True),
    dict(doc=True, causal=True),
    dict(causal=True, window=150),
    dict(window=97),
    dict(prefix_len=77),
    dict(prefix_len=200, window=130),
    dict(doc=True, causal=True, window=64),
    dict(doc=True, prefix_len=40),
]
SCORES = [dict(), dict(alibi=True), dict(softcap=20.0), dict(alibi=True, softcap=30.0)]


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("si", range(len(SCORES)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_cases(ci, si, dtype):
    kw = dict(CASES[ci])
    kw.update(SCORES[si])
    # Ragged lengths, Lq != Lkv only without self-attention-only structure, GQA 4:2.
    Lq, Lkv = (333, 333) if kw.get("doc") else (333, 401)
    w = random_case(10 * ci + si, dtype=dtype, B=2, Hq=4, Hkv=2, Lq=Lq, Lkv=Lkv, **kw)
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w))
    blocks = [(128, 128), (128, 64)] + ([(256, 64), (256, 128)] if dtype == "bf16" else [])
    for qb, kvb in blocks:
        out, lse, _ = run_gpu(w, kv_block=kvb, q_block=qb)
        check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, dtype,
                    f"case {ci}/{si}/{dtype}/q{qb}/kv{kvb}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_null_block_mask_dense(dtype):
    w = random_case(501, dtype=dtype, B=1, Hq=8, Hkv=1, Lq=200, Lkv=300)
    out, lse, _ = run_gpu(w, use_bm=False)
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, {})
    check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, dtype, "null bm")


@pytest.mark.parametrize("Lkv", [1, 40, 64, 65, 128, 129, 191, 192, 256, 257, 320, 383, 384, 449, 1000])
@pytest.mark.parametrize("si", range(len(SCORES)))
def test_null_block_mask_bf16_pipelined(Lkv, si):
    """bf16 without a BlockMask runs the software-pipelined every-tile-full kernel: one to eight and
    sixteen 64-key steps (from three steps on the two wave groups run alternating phases, with one
    or two steps after them), exact and ragged last steps, every score transform, GQA 6:2, B = 2."""
    kw = dict(SCORES[si])
    w = random_case(5000 + 7 * Lkv + si, dtype="bf16", B=2, Hq=6, Hkv=2, Lq=150, Lkv=Lkv, **kw)
    out, lse, _ = run_gpu(w, use_bm=False)
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w))
    check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16", f"null bm Lkv {Lkv} score {si}")


@pytest.mark.parametrize("Lkv", [1, 40, 64, 65, 128, 129, 191, 192, 257])
@pytest.mark.parametrize("kw", [dict(causal=True, softcap=20.0), dict(window=97, alibi=True), dict()])
def test_interval_masks_bf16_pipelined_short_rows(Lkv, kw):
    """bf16 with a 128-query BlockMask and a mask without document ids runs the software-pipelined
    block-sparse kernel: lists of one to five 64-key steps (64- and 128-key tiles), exact and
    ragged last tiles, halves of 128-key tiles past the last key, GQA 4:2."""
    w = random_case(5200 + 7 * Lkv + len(kw), dtype="bf16", B=1, Hq=4, Hkv=2, Lq=150, Lkv=Lkv, **kw)
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w))
    for kvb in (64, 128):
        out, lse, _ = run_gpu(w, kv_block=kvb, q_block=128)
        check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16",
                    f"interval masks Lkv {Lkv} {sorted(kw)} kv{kvb}")


def test_null_block_mask_bf16_strided_and_scale():
    import torch
    fa = _fa()
    w = random_case(5100, dtype="bf16", B=2, Hq=4, Lq=333, Lkv=333)
    dev = torch.device("cuda", 0)
    q, k, v = (to_device(x, "bf16", dev).transpose(1, 2).contiguous().transpose(1, 2) for x in (w.q, w.k, w.v))
    out, lse = fa.flexattn_fwd(q, k, v, None, fa.FA_MASK_NONE, sm_scale=0.03)
    torch.cuda.synchronize()
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, dict(sm_scale=0.03))
    check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16", "null bm strided")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fully_masked_rows_and_empty_rows(dtype):
    # Unsorted document ids with query ids absent from the keys: those rows have no allowed
    # key (out 0, lse -inf); a whole query block with none gives an empty BlockMask row.
    w = random_case(502, dtype=dtype, B=1, Hq=2, Lq=300, Lkv=300, doc=True, n_docs=4, doc_sorted=False)
    w.q_doc = w.q_doc.copy()
    w.q_doc[0, 5] = 99
    w.q_doc[0, 256:] = 77
    out, lse, bm = run_gpu(w)
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w))
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    if dtype == "bf16":  # the same with 256-query workgroups (a whole 256-query row empty)
        w2 = random_case(503, dtype=dtype, B=1, Hq=2, Lq=600, Lkv=600, doc=True, n_docs=4, doc_sorted=False)
        w2.q_doc = w2.q_doc.copy()
        w2.q_doc[0, 256:512] = 77
        out2, lse2, bm2 = run_gpu(w2, q_block=256, kv_block=64)
        qf2, kf2, vf2 = w2.qkv_f32()
        o_ref2, l_ref2 = ref_attn.attention(qf2, kf2, vf2, spec_of(w2))
        assert int(bm2.kv_num_blocks[0, 0, 1]) == 0 and int(bm2.full_kv_num_blocks[0, 0, 1]) == 0
        check_close(out2.float().cpu().numpy(), lse2.cpu().numpy(), o_ref2, l_ref2, dtype, "masked rows q256")
    assert np.all(o[0, :, 5] == 0) and np.all(np.isneginf(l[0, :, 5]))
    assert np.all(o[0, :, 256:] == 0) and np.all(np.isneginf(l[0, :, 256:]))
    assert int(bm.kv_num_blocks[0, 0, 2]) == 0 and int(bm.full_kv_num_blocks[0, 0, 2]) == 0
    check_close(o, l, o_ref, l_ref, dtype, "masked rows")


def test_gqa_ratios_and_strided_views():
    import torch
    fa = _fa()
    for Hq, Hkv in [(8, 8), (8, 4), (8, 2), (8, 1)]:
        w = random_case(600 + Hq * 10 + Hkv, dtype="bf16", B=1, Hq=Hq, Hkv=Hkv, Lq=260, causal=True)
        out, lse, _ = run_gpu(w, q_block=256 if Hkv % 2 == 0 else 128, kv_block=64)
        qf, kf, vf = w.qkv_f32()
        o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w))
        check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16", f"gqa {Hq}/{Hkv}")
    # Non-contiguous [B, L, H, D] storage viewed as [B, H, L, D].
    w = random_case(650, dtype="bf16", B=2, Hq=4, Lq=190, causal=True)
    dev = torch.device("cuda", 0)
    q, k, v = (to_device(x, "bf16", dev).transpose(1, 2).contiguous().transpose(1, 2) for x in (w.q, w.k, w.v))
    assert q.stride(2) == 4 * 128
    bm = fa.flexattn_block_mask_build(fa.FA_MASK_CAUSAL, 2, 190, 190)
    out, lse = fa.flexattn_fwd(q, k, v, bm, fa.FA_MASK_CAUSAL)
    torch.cuda.synchronize()
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w))
    check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16", "strided")


def test_empty_inputs():
    import torch
    fa = _fa()
    dev = torch.device("cuda", 0)
    q = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    k = torch.randn((1, 2, 50, 128), device=dev).bfloat16()
    out, lse = fa.flexattn_fwd(q, k, k, None, fa.FA_MASK_NONE)
    assert out.shape == (1, 2, 0, 128)
    q = torch.randn((1, 2, 70, 128), device=dev).bfloat16()
    k0 = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    out, lse = fa.flexattn_fwd(q, k0, k0, None, fa.FA_MASK_NONE)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_sm_scale_override():
    w = random_case(700, dtype="f32", B=1, Hq=2, Lq=150, causal=True)
    import torch
    fa = _fa()
    dev = torch.device("cuda", 0)
    q, k, v = (to_device(x, "f32", dev) for x in (w.q, w.k, w.v))
    bm = fa.flexattn_block_mask_build(fa.FA_MASK_CAUSAL, 1, 150, 150)
    out, lse = fa.flexattn_fwd(q, k, v, bm, fa.FA_MASK_CAUSAL, sm_scale=0.05)
    torch.cuda.synchronize()
    o_ref, l_ref = ref_attn.attention(w.q, w.k, w.v, dict(causal=True, sm_scale=0.05))
    check_close(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "f32", "sm_scale")


# ------------------------------- full-size workloads ----------------------------------------

def _sample_rows(w, rng, n_heads=3, n_rows=96):
    """(b, hq, rows): first and last rows, the ragged tail and random rows."""
    out = []
    for _ in range(n_heads):
        b = int(rng.integers(w.B))
        hq = int(rng.integers(w.Hq))
        rows = set(rng.integers(0, w.Lq, n_rows).tolist()) | {0, 1, w.Lq - 1, w.Lq - 2}
        rows |= set(range(max(0, (w.Lq // 128) * 128 - 3), min(w.Lq, (w.Lq // 128) * 128 + 3)))
        out.append((b, hq, np.array(sorted(rows))))
    return out


@pytest.mark.parametrize("name", [
    "grouped_variate_4x17_f32",
    "grouped_variate_4096g_bf16",
    "doc_causal_b4h16t8192_bf16",
    "swa1024_gqa32x8_softcap50_t16384_bf16",
    "dense_b1h32s24576_bf16",
])
@pytest.mark.parametrize("blocks", ["bench", "128x128"])
def test_workloads_full_size(name, blocks):
    """blocks="bench": the launch configuration bench.py times (BENCH_BLOCKS); else 128x128."""
    print(f"workload {name} blocks {blocks}", flush=True)
    w = make_workload(name)
    qb, kvb = (128, 128) if blocks != "bench" else BENCH_BLOCKS[w.dtype]
    out, lse, bm = run_gpu(w, q_block=qb, kv_block=kvb)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    del out, lse
    qf, kf, vf = w.qkv_f32()
    spec = spec_of(w)
    if name == "grouped_variate_4x17_f32":
        o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec)
        check_close(o, l, o_ref, l_ref, w.dtype, name)
        return
    if name == "grouped_variate_4096g_bf16":
        o_ref, l_ref = ref_attn.attention_by_groups(qf, kf, vf, w.q_doc)
        check_close(o, l, o_ref, l_ref, w.dtype, name + " (all rows, per group)")
    rng = np.random.default_rng(123)
    got, want, gl, wl = [], [], [], []
    for b, hq, rows in _sample_rows(w, rng):
        orow, lrow = ref_attn.attention_rows(qf, kf, vf, spec, b, hq, rows)
        got.append(o[b, hq, rows])
        want.append(orow)
        gl.append(l[b, hq, rows])
        wl.append(lrow)
    check_close(np.concatenate(got), np.concatenate(gl), np.concatenate(want), np.concatenate(wl), w.dtype,
                name + " (sampled rows)")
    # Property at any size: every output row is a convex combination of V rows, so it lies in
    # the per-channel range of V.
    vmin = vf.min(axis=2).min()
    vmax = vf.max(axis=2).max()
    assert np.isfinite(o).all() and o.min() >= vmin - 1e-2 and o.max() <= vmax + 1e-2


@pytest.mark.parametrize("kw", [dict(doc=True, causal=True), dict(causal=True, window=300, alibi=True)])
def test_f32_both_launch_shapes(kw):
    """fp32 inputs with fewer than 256 work items run the split-key kernel (four workgroups per
    work item, keys split over the waves); larger ones the one-workgroup kernel. Both against
    the oracle: B=2, 16 heads, 1100 queries is 288 work items; one head of it is 9."""
    w = random_case(610, dtype="f32", B=2, Hq=16, Hkv=8, Lq=1100, Lkv=1100, **kw)
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w))
    out, lse, _ = run_gpu(w)
    check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "f32", "f32 288 work items")
    w1 = random_case(611, dtype="f32", B=1, Hq=1, Hkv=1, Lq=1100, Lkv=1100, **kw)
    qf, kf, vf = w1.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w1))
    out, lse, _ = run_gpu(w1)
    check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "f32", "f32 9 work items")

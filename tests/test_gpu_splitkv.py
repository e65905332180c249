"""GPU: the split-KV forward (decoding form) matches the fp64 oracle for every split count,
including more splits than tiles (empty ranges), GQA (also with the query heads of a kv head
packed into one workgroup), masks and score mods."""
import numpy as np
import pytest

from oracle import attention as ref_attn
from tests._util import check_close, to_device
from workloads import random_case

pytestmark = pytest.mark.gpu

CASES = [
    # (seed, kwargs, mask description)
    (11, dict(B=2, Hq=8, Hkv=2, Lq=1, Lkv=3000), "none"),
    (12, dict(B=1, Hq=4, Lq=16, Lkv=2000, doc=True, n_docs=3), "doc"),
    (13, dict(B=1, Hq=4, Hkv=2, Lq=16, Lkv=1500, window=600, softcap=30.0, alibi=True), "window+softcap+alibi"),
    (14, dict(B=1, Hq=2, Lq=300, Lkv=900, causal=True), "causal, several query blocks"),
    (15, dict(B=1, Hq=2, Lq=5, Lkv=500), "few tiles"),
    # grouped query heads packed into one workgroup per kv head (group * Lq <= 128)
    (16, dict(B=1, Hq=6, Hkv=2, Lq=7, Lkv=1200, doc=True, n_docs=2), "packed GQA, doc"),
    (17, dict(B=2, Hq=8, Hkv=2, Lq=16, Lkv=900, causal=True, softcap=20.0), "packed GQA, causal+softcap"),
    (18, dict(B=1, Hq=16, Hkv=2, Lq=16, Lkv=700, alibi=True), "packed GQA, 8 heads x 16 queries"),
]


def _fa():
    import block_sparse_masked_blockmask_amd as fa
    return fa


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("n_splits", [1, 4, 64])
def test_splitkv_matches_oracle(ci, n_splits):
    import torch
    fa = _fa()
    seed, kw, what = CASES[ci]
    w = random_case(seed, dtype="bf16", **kw)
    print(f"case: splitkv {what} n_splits={n_splits}", flush=True)
    dev = torch.device("cuda", 0)
    q, k, v = (to_device(x, "bf16", dev) for x in (w.q, w.k, w.v))
    mk = (fa.FA_MASK_DOC if w.doc else 0) | (fa.FA_MASK_CAUSAL if w.causal else 0) \
        | (fa.FA_MASK_WINDOW if w.window is not None else 0)
    sk = (fa.FA_SCORE_ALIBI if w.alibi_slopes is not None else 0) | (fa.FA_SCORE_SOFTCAP if w.softcap else 0)
    qd = kd = sl = None
    if w.doc:
        qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
        kd = torch.from_numpy(np.ascontiguousarray(w.kv_doc)).to(dev)
    if w.alibi_slopes is not None:
        sl = torch.from_numpy(w.alibi_slopes).to(dev)
    bm = None
    if mk:
        bm = fa.flexattn_block_mask_build(mk, w.B, w.Lq, w.Lkv, 128, 64, q_doc=qd, kv_doc=kd,
                                          window=w.window or 0, device=dev)
    out, lse = fa.flexattn_fwd_splitkv(q, k, v, bm, mk, sk, n_splits=n_splits, window=w.window or 0,
                                       softcap=w.softcap or 0.0, alibi_slopes=sl, q_doc=qd, kv_doc=kd)
    torch.cuda.synchronize()
    qf, kf, vf = w.qkv_f32()
    spec = dict(doc=w.doc, causal=w.causal, window=w.window, q_doc=w.q_doc, kv_doc=w.kv_doc,
                alibi_slopes=w.alibi_slopes, softcap=w.softcap)
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec)
    check_close(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16", f"splitkv {what} {n_splits}")

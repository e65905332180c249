"""GPU: the optional BlockMask schedule (row_order).

The device builder's schedule is bit-exact with the host builder's, and a forward that uses
it is bit-identical to one that does not (each work item's arithmetic does not depend on
when it runs), on small cases of every mask and at the workloads' full sizes.
"""
import numpy as np
import pytest

from oracle import attention as ref_attn
from tests._util import check_close, to_device
from tests.test_gpu_fwd import BENCH_BLOCKS, mask_kind, score_kind, spec_of
from workloads import make_workload, random_case

pytestmark = pytest.mark.gpu

CASES = [
    dict(),
    dict(causal=True),
    dict(doc=True),
    dict(doc=True, causal=True),
    dict(causal=True, window=150, softcap=20.0),
    dict(prefix_len=77, alibi=True),
    dict(doc=True, causal=True, window=64),
]


def _run(w, q_block, kv_block, row_order):
    import torch
    import block_sparse_masked_blockmask_amd as fa
    dev = torch.device("cuda", 0)
    q, k, v = (to_device(x, w.dtype, dev) for x in (w.q, w.k, w.v))
    qd = kd = sl = None
    if w.doc:
        qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
        kd = torch.from_numpy(np.ascontiguousarray(w.kv_doc)).to(dev)
    if w.alibi_slopes is not None:
        sl = torch.from_numpy(w.alibi_slopes).to(dev)
    mk, sk = mask_kind(w), score_kind(w)
    bm = fa.flexattn_block_mask_build(mk, w.B, w.Lq, w.Lkv, q_block, kv_block, q_doc=qd, kv_doc=kd,
                                      window=w.window or 0, prefix_len=w.prefix_len or 0, device=dev,
                                      row_order=row_order)
    out, lse = fa.flexattn_fwd(q, k, v, bm, mk, sk, window=w.window or 0, prefix_len=w.prefix_len or 0,
                               softcap=w.softcap or 0.0, alibi_slopes=sl, q_doc=qd, kv_doc=kd)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), bm


def _host_order(w, q_block, kv_block):
    import block_sparse_masked_blockmask_amd as fa
    mk = mask_kind(w)
    qd = np.ascontiguousarray(w.q_doc, np.int32) if w.doc else None
    kd = np.ascontiguousarray(w.kv_doc, np.int32) if w.doc else None
    bm = fa.flexattn_block_mask_build_host(mk, w.B, w.Lq, w.Lkv, q_block, kv_block, q_doc=qd, kv_doc=kd,
                                           window=w.window or 0, prefix_len=w.prefix_len or 0, row_order=True)
    return bm.row_order.numpy()


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ordered_forward_small(ci, dtype):
    kw = dict(CASES[ci])
    Lq, Lkv = (1333, 1333) if kw.get("doc") else (1333, 1401)
    w = random_case(4000 + ci, dtype=dtype, B=2, Hq=4, Hkv=2, Lq=Lq, Lkv=Lkv, **kw)
    blocks = [(128, 128), (128, 64)] + ([(256, 64)] if dtype == "bf16" else [])
    for qb, kvb in blocks:
        o0, l0, _ = _run(w, qb, kvb, False)
        o1, l1, bm = _run(w, qb, kvb, True)
        assert np.array_equal(bm.row_order.cpu().numpy(), _host_order(w, qb, kvb)), (qb, kvb)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1), (qb, kvb)
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, spec_of(w))
    check_close(o1, l1, o_ref, l_ref, dtype, f"ordered case {ci}/{dtype}")


@pytest.mark.parametrize("name", [
    "grouped_variate_4096g_bf16",
    "doc_causal_b4h16t8192_bf16",
    "swa1024_gqa32x8_softcap50_t16384_bf16",
])
def test_ordered_forward_workloads(name):
    print(f"workload {name}", flush=True)
    w = make_workload(name)
    qb, kvb = BENCH_BLOCKS[w.dtype]
    o0, l0, _ = _run(w, qb, kvb, False)
    o1, l1, bm = _run(w, qb, kvb, True)
    assert np.array_equal(bm.row_order.cpu().numpy(), _host_order(w, qb, kvb))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)

"""GPU: the group-count sweep of the grouped variate workload (8/32/64/128 groups of 17
variates, H=4, D=128, fp32 and bf16). Both the block-sparse BlockMask and an all-live BlockMask
(every tile partial, the dense-iteration baseline) go through the same kernel and must match the
fp64 oracle on the whole output."""
import numpy as np
import pytest

from oracle import attention as ref_attn
from tests._util import check_close, to_device
from workloads import SWEEP_GROUPS, grouped_sweep

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_groups", SWEEP_GROUPS)
def test_sweep_sparse_and_all_live_match_oracle(n_groups, dtype):
    import torch
    import block_sparse_masked_blockmask_amd as fa
    w = grouped_sweep(n_groups, dtype)
    print(f"case: sweep groups={n_groups} dtype={dtype} L={w.Lq}", flush=True)
    dev = torch.device("cuda", 0)
    q, k, v = (to_device(x, w.dtype, dev) for x in (w.q, w.k, w.v))
    qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
    kv_block = 64 if dtype == "bf16" else 128
    sparse = fa.flexattn_block_mask_build(fa.FA_MASK_DOC, 1, w.Lq, w.Lkv, 128, kv_block, q_doc=qd, kv_doc=qd)
    dense = fa.block_mask_all_partial(1, 1, w.Lq, w.Lkv, 128, kv_block, device=dev)
    qf, kf, vf = w.qkv_f32()  # the exact values the GPU receives (bf16 bit patterns widened)
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, dict(doc=True, q_doc=w.q_doc, kv_doc=w.kv_doc))
    for bm in (sparse, dense):
        out, lse = fa.flexattn_fwd(q, k, v, bm, fa.FA_MASK_DOC, q_doc=qd, kv_doc=qd)
        torch.cuda.synchronize()
        o = out.float().cpu().numpy() if dtype == "bf16" else out.cpu().numpy()
        check_close(o, lse.cpu().numpy(), o_ref, l_ref, dtype, f"sweep {n_groups} {dtype}")
    n_sparse = int(sparse.kv_num_blocks.sum() + sparse.full_kv_num_blocks.sum())
    assert n_sparse <= dense.n_qb * dense.n_kvb

"""GPU: the BlockMask build and the forward can be captured in a HIP graph.

The C ABI allocates nothing and never synchronises, so a caller can capture a whole step
(BlockMask build + forward) once and replay it. Each replay is checked against the eager
result, with eager work and host synchronisation between replays, and with the inputs
changed in place between replays (a replay must read the buffers, not reuse old results).
"""
import numpy as np
import pytest

from tests._util import to_device
from tests.test_gpu_fwd import mask_kind, score_kind
from workloads import random_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kw,row_order", [
    (dict(doc=True, causal=True), True),
    (dict(doc=True), False),
    (dict(causal=True, window=200, softcap=30.0), False),
])
def test_captured_step_replays(kw, row_order):
    import torch
    import block_sparse_masked_blockmask_amd as fa
    dev = torch.device("cuda", 0)
    w = random_case(5100, dtype="bf16", B=2, Hq=4, Hkv=2, Lq=1500, Lkv=1500, **kw)
    q, k, v = (to_device(x, w.dtype, dev) for x in (w.q, w.k, w.v))
    qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev) if w.doc else None
    mk, sk = mask_kind(w), score_kind(w)
    bm = fa.BlockMask(w.B if w.doc else 1, 1, w.Lq, w.Lkv, 128, 64, dev, row_order=row_order)
    wsb = fa.flexattn_block_mask_workspace_bytes(mk, w.B, w.Lq, w.Lkv, 128, 64)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def step():
        s = torch.cuda.current_stream()
        fa.flexattn_block_mask_build(mk, w.B, w.Lq, w.Lkv, 128, 64, q_doc=qd, kv_doc=qd, window=w.window or 0,
                                     out=bm, workspace=ws, stream=s)
        fa.flexattn_fwd(q, k, v, bm, mk, sk, window=w.window or 0, softcap=w.softcap or 0.0, q_doc=qd,
                        kv_doc=qd, out=out, lse=lse, stream=s)

    def eager_result():
        step()
        torch.cuda.synchronize()
        return out.clone(), lse.clone()

    ref_o, ref_l = eager_result()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {r}"
        # eager work between replays
        ref_o2, _ = eager_result()
        assert torch.equal(ref_o2, ref_o)
    # Inputs changed in place: the replay recomputes from the new values.
    q.mul_(0.5)
    new_o, new_l = eager_result()
    out.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, new_o) and torch.equal(lse, new_l)
    assert not torch.equal(new_l, ref_l)

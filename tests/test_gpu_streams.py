"""GPU: calls on a side stream with temporaries allocated by the binding.

The binding allocates workspaces (and outputs when none are given) with the caching allocator
on the current stream, while the kernels run on the stream passed in. It records those tensors
on the launch stream, so their memory is not handed to another allocation on the current stream
while the side stream's kernels may still use it. Each case below allocates and overwrites
fresh memory on the current stream right after the call (where a missing record would let the
allocator reuse the workspace) and compares the side-stream results with current-stream ones.
"""
import numpy as np
import pytest

from tests._util import to_device
from workloads import grad_output, random_case

pytestmark = pytest.mark.gpu


def _scribble(torch, dev, nbytes):
    """Allocate and overwrite memory on the current stream (reuses freed blocks if allowed)."""
    junk = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(0xA5) for _ in range(4)]
    return junk


def test_side_stream_temporaries_match_current_stream():
    import torch
    import block_sparse_masked_blockmask_amd as fa
    dev = torch.device("cuda", 0)
    w = random_case(4242, dtype="bf16", B=2, Hq=4, Hkv=2, Lq=1500, doc=True, causal=True, n_docs=12)
    q, k, v = (to_device(x, "bf16", dev) for x in (w.q, w.k, w.v))
    qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
    mk = fa.FA_MASK_DOC | fa.FA_MASK_CAUSAL
    do = to_device(grad_output(w, 4242), "bf16", dev)

    def run(stream):
        bm = fa.flexattn_block_mask_build(mk, w.B, w.Lq, w.Lkv, 128, 128, q_doc=qd, kv_doc=qd, stream=stream)
        out, lse = fa.flexattn_fwd(q, k, v, bm, mk, q_doc=qd, kv_doc=qd, stream=stream)
        o_kv, l_kv = fa.flexattn_fwd_splitkv(q, k, v, bm, mk, n_splits=4, q_doc=qd, kv_doc=qd, stream=stream)
        grads = fa.flexattn_bwd(q, k, v, out, do, lse, bm, None, mk, q_doc=qd, kv_doc=qd, stream=stream)
        qz = fa.flexattn_quantize_qkv_ex(q, k, k, qk_block=32, center_k=True, stream=stream)
        oq, lq = fa.flexattn_fwd_quant(qz, stream=stream)
        return [bm.kv_indices, bm.full_kv_indices, out, lse, o_kv, l_kv, *grads[:3], qz["k8"], qz["k_mean"], oq, lq]

    ref = [t.clone() for t in run(None)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        got = run(side)
        junk = _scribble(torch, dev, 8 << 20)  # the current stream reuses whatever the allocator allows
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, i)
        del junk, got

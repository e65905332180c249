"""GPU: the FLEXATTN_VERIFY_BLOCKMASK debug mode.

With the variable set, the forward and the backward copy the BlockMask lists to the host and
check them before enqueuing anything. A valid BlockMask gives the same results as without the
check; a corrupted one is refused with FA_ERR_INVALID_ARG naming the row (no kernel runs on it).
"""
import numpy as np
import pytest

from tests._util import to_device
from workloads import grad_output, random_case

pytestmark = pytest.mark.gpu


def _setup():
    import torch
    import block_sparse_masked_blockmask_amd as fa
    dev = torch.device("cuda", 0)
    w = random_case(77, dtype="bf16", B=2, Hq=2, Lq=700, doc=True, causal=True, n_docs=6)
    q, k, v = (to_device(x, "bf16", dev) for x in (w.q, w.k, w.v))
    qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
    mk = fa.FA_MASK_DOC | fa.FA_MASK_CAUSAL
    bm = fa.flexattn_block_mask_build(mk, 2, 700, 700, 128, 128, q_doc=qd, kv_doc=qd)
    return torch, fa, w, q, k, v, qd, mk, bm


def test_valid_block_mask_passes_unchanged(monkeypatch):
    torch, fa, w, q, k, v, qd, mk, bm = _setup()
    o0, l0 = fa.flexattn_fwd(q, k, v, bm, mk, q_doc=qd, kv_doc=qd)
    do = to_device(grad_output(w, 77), "bf16", q.device)
    g0 = fa.flexattn_bwd(q, k, v, o0, do, l0, bm, None, mk, q_doc=qd, kv_doc=qd)
    monkeypatch.setenv("FLEXATTN_VERIFY_BLOCKMASK", "1")
    o1, l1 = fa.flexattn_fwd(q, k, v, bm, mk, q_doc=qd, kv_doc=qd)
    g1 = fa.flexattn_bwd(q, k, v, o1, do, l1, bm, None, mk, q_doc=qd, kv_doc=qd)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0[:3], g1[:3]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("corrupt,needle", [
    ("count_high", "counts"),
    ("count_negative", "counts"),
    ("entry_range", "outside"),
    ("not_ascending", "ascending"),
    ("full_and_partial", "both full and partial"),
])
def test_corrupt_block_mask_is_refused(monkeypatch, corrupt, needle):
    torch, fa, w, q, k, v, qd, mk, bm = _setup()
    out = torch.full(q.shape, 7.0, dtype=q.dtype, device=q.device)
    n = bm.n_kvb
    row = (1, 0, 4)  # batch 1, query block 4: two partial tiles (3, 4) in this case
    assert int(bm.kv_num_blocks[row]) >= 2, int(bm.kv_num_blocks[row])
    if corrupt == "count_high":
        bm.kv_num_blocks[row] = n + 1
    elif corrupt == "count_negative":
        bm.full_kv_num_blocks[row] = -1
    elif corrupt == "entry_range":
        bm.kv_indices[row + (0,)] = n
    elif corrupt == "not_ascending":
        a, b = int(bm.kv_indices[row + (0,)]), int(bm.kv_indices[row + (1,)])
        bm.kv_indices[row + (0,)], bm.kv_indices[row + (1,)] = b, a
    else:
        # The full list becomes exactly the first partial block: ascending, but listed twice.
        bm.full_kv_indices[row + (0,)] = int(bm.kv_indices[row + (0,)])
        bm.full_kv_num_blocks[row] = 1
    monkeypatch.setenv("FLEXATTN_VERIFY_BLOCKMASK", "1")
    with pytest.raises(fa.FlexAttnError) as e:
        fa.flexattn_fwd(q, k, v, bm, mk, q_doc=qd, kv_doc=qd, out=out)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and needle in e.value.reason and "row" in e.value.reason
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "the refused call wrote its output"

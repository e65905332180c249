"""GPU: whole-output parity of the full-size workloads, in the launch configuration bench.py times.

Every case runs through bench.Case (the bench's own BlockMask build and forward calls) and is
compared against the fp64 oracle:
  - the BlockMask at the timed 128 x 64 tiling, bit-exact on every row (the 4096-group workload
    in two halves of its 1,051 rows);
  - causal document packing (B=4, H=16, T=8192) on its whole output, through the per-document
    causal restatement of the oracle (pinned against the definition and causal SDPA);
  - sliding-window GQA with soft-cap (B=2, 32/8 heads, T=16384) on its whole output, one batch
    per test, through the banded restatement (pinned the same way);
  - dense B=1, H=32, S=24576 bf16 on one whole head (24,576 rows against all keys);
  - the int8/fp8 form of the dense workload: every code and scale of Q8, K8 and V8 bit-exact, and
    the cosine gate over one whole head.
"""
import numpy as np
import pytest

import bench
from oracle import attention as ref_attn
from oracle import blockmask as ref_bm
from oracle import quant as ref_q
from tests._util import check_close, cosine
from workloads import make_workload

pytestmark = pytest.mark.gpu

KEYS = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")


def _run(w, quantized=False):
    """One bench step (BlockMask build or quantization, then the forward) on cuda:0; returns the
    finished Case (outputs still on the device)."""
    import torch
    import block_sparse_masked_blockmask_amd as fa
    case = bench.Case(fa, torch, torch.device("cuda", 0), w, quantized=quantized)
    case.step()
    torch.cuda.synchronize()
    return case


def _spec(w):
    return dict(doc=w.doc, causal=w.causal, window=w.window, prefix_len=w.prefix_len, q_doc=w.q_doc, kv_doc=w.kv_doc)


@pytest.mark.parametrize("name,part", [
    ("grouped_variate_4096g_bf16", 0),
    ("grouped_variate_4096g_bf16", 1),
    ("doc_causal_b4h16t8192_bf16", None),
    ("swa1024_gqa32x8_softcap50_t16384_bf16", None),
])
def test_block_mask_at_bench_tiling_every_row(name, part):
    print(f"block mask {name} part {part}", flush=True)
    w = make_workload(name)
    case = _run(w)
    L = case.launch
    assert (L["q_block"], L["kv_block"]) == (128, 64) and case.bm is not None
    got = {k: getattr(case.bm, k).cpu().numpy() for k in KEYS}
    Bm = w.B if w.doc else 1
    nqb = -(-w.Lq // 128)
    rows = [(b, qb) for b in range(Bm) for qb in range(nqb)]
    if part is not None:
        half = (len(rows) + 1) // 2
        rows = rows[part * half:(part + 1) * half]
    ref = ref_bm.block_mask(_spec(w), w.B, w.Lq, w.Lkv, 128, 64, rows=rows)
    for bm, qb in rows:
        for k in ("kv_num_blocks", "full_kv_num_blocks"):
            assert got[k][bm, 0, qb] == ref[k][bm, 0, qb], (k, bm, qb)
        for k in ("kv_indices", "full_kv_indices"):
            assert np.array_equal(got[k][bm, 0, qb], ref[k][bm, 0, qb]), (k, bm, qb)
    if L["row_order"]:
        # The schedule is a permutation of the query blocks of every row set.
        order = case.bm.row_order.cpu().numpy()
        for bm in range(Bm):
            assert sorted(order[bm, 0].tolist()) == list(range(nqb))
    if name.startswith("swa1024"):
        # Closed form at 64-key blocks: per row, every key block within the window is full except
        # the diagonal block(s) and the two window edges.
        nf, np_ = int(got["full_kv_num_blocks"].sum()), int(got["kv_num_blocks"].sum())
        print(f"{name}: full {nf}, partial {np_}")


def test_doc_causal_whole_output():
    print("doc_causal_b4h16t8192_bf16 whole output", flush=True)
    w = make_workload("doc_causal_b4h16t8192_bf16")
    case = _run(w)
    assert case.launch["row_order"] and case.launch["kv_block"] == 64
    o = case.out.float().cpu().numpy()
    l = case.lse.cpu().numpy()
    del case
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention_by_documents_causal(qf, kf, vf, w.q_doc)
    check_close(o, l, o_ref, l_ref, "bf16", "doc-causal (every row, per document)")


@pytest.mark.parametrize("b", [0, 1])
def test_swa_softcap_whole_output(b):
    print(f"swa1024_gqa32x8_softcap50_t16384_bf16 whole output, batch {b}", flush=True)
    w = make_workload("swa1024_gqa32x8_softcap50_t16384_bf16")
    case = _run(w)
    o = case.out[b].float().cpu().numpy()
    l = case.lse[b].cpu().numpy()
    del case
    qf, kf, vf = w.qkv_f32()
    heads = [(b, h) for h in range(w.Hq)]
    o_ref, l_ref = ref_attn.attention_band(qf, kf, vf, w.window, softcap=w.softcap, heads=heads)
    check_close(o, l, o_ref[b], l_ref[b], "bf16", f"sliding window + soft-cap, batch {b} (every row)")


def test_dense_whole_head():
    print("dense_b1h32s24576_bf16 whole head", flush=True)
    w = make_workload("dense_b1h32s24576_bf16")
    case = _run(w)
    hq = 17
    o = case.out[0, hq].float().cpu().numpy()
    l = case.lse[0, hq].cpu().numpy()
    del case
    qf, kf, vf = w.qkv_f32()
    o_ref = np.empty_like(o, dtype=np.float64)
    l_ref = np.empty(l.shape, np.float64)
    for r0 in range(0, w.Lq, 2048):
        rows = np.arange(r0, min(w.Lq, r0 + 2048))
        o_ref[rows], l_ref[rows] = ref_attn.attention_rows(qf, kf, vf, {}, 0, hq, rows)
    check_close(o, l, o_ref, l_ref, "bf16", f"dense head {hq} (every row)")


def test_dense_quantized_codes_and_whole_head():
    print("dense_b1h32s24576_bf16 quantized: all codes, whole head", flush=True)
    w = make_workload("dense_b1h32s24576_bf16")
    case = _run(w, quantized=True)
    qb = case.qbufs
    got = {k: qb[k].cpu().numpy() for k in ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale")}
    hq = 5
    o = case.out[0, hq].float().cpu().numpy()
    del case, qb
    qf, kf, vf = w.qkv_f32()
    for h in range(w.Hq):  # every head, one at a time (the oracle's quantizers in float32)
        c, s = ref_q.quantize_int8_blocks(qf[:, h:h + 1])
        assert np.array_equal(got["q8"][:, h:h + 1], c) and np.array_equal(got["q_scale"][:, h:h + 1], s), ("q", h)
        c, s = ref_q.quantize_int8_blocks(kf[:, h:h + 1])
        assert np.array_equal(got["k8"][:, h:h + 1], c) and np.array_equal(got["k_scale"][:, h:h + 1], s), ("k", h)
        c, s = ref_q.quantize_fp8_channels(vf[:, h:h + 1])
        assert np.array_equal(got["v8"][:, h:h + 1], c) and np.array_equal(got["v_scale"][:, h:h + 1], s), ("v", h)
    o_ref = np.empty(o.shape, np.float64)
    for r0 in range(0, w.Lq, 2048):
        rows = np.arange(r0, min(w.Lq, r0 + 2048))
        o_ref[rows], _ = ref_attn.attention_rows(qf, kf, vf, {}, 0, hq, rows)
    c = cosine(o, o_ref)
    print(f"quantized cosine over head {hq} (24576 rows) vs the unquantized oracle: {c:.6f}")
    assert c >= 0.999, c

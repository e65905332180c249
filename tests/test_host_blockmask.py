"""The host BlockMask builder (C ABI, no GPU) is bit-exact with the exhaustive oracle.

The host builder shares its closed forms with the device builder, so these CPU tests also cover
the classification logic the GPU runs.
"""
import numpy as np
import pytest

from oracle import blockmask as ref_bm
from workloads import random_case

KEYS = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")

SPECS = [
    {}, {"causal": True}, {"window": 37}, {"causal": True, "window": 100}, {"prefix_len": 77},
    {"prefix_len": 50, "window": 90}, {"doc": True}, {"doc": True, "causal": True},
    {"doc": True, "causal": True, "window": 64}, {"doc": True, "prefix_len": 30},
]


def _fa():
    import block_sparse_masked_blockmask_amd as fa
    fa.lib()
    return fa


def _mask_kind(fa, spec):
    m = fa.FA_MASK_DOC if spec.get("doc") else 0
    m |= fa.FA_MASK_CAUSAL if spec.get("causal") else 0
    m |= fa.FA_MASK_WINDOW if spec.get("window") is not None else 0
    m |= fa.FA_MASK_PREFIX_LM if spec.get("prefix_len") is not None else 0
    return m


def build_host(spec, B, Lq, Lkv, BQ, BK):
    fa = _fa()
    qd = kd = None
    if spec.get("doc"):
        qd = np.ascontiguousarray(spec["q_doc"], np.int32)
        kd = np.ascontiguousarray(spec["kv_doc"], np.int32)
    bm = fa.flexattn_block_mask_build_host(_mask_kind(fa, spec), B, Lq, Lkv, BQ, BK, q_doc=qd, kv_doc=kd,
                                           window=spec.get("window") or 0, prefix_len=spec.get("prefix_len") or 0)
    return {k: getattr(bm, k).numpy() for k in KEYS}


@pytest.mark.parametrize("si", range(len(SPECS)))
@pytest.mark.parametrize("shape", [(2, 333, 333, 128, 128), (1, 700, 517, 64, 128), (2, 260, 390, 128, 64),
                                   (1, 64, 64, 64, 64), (2, 600, 600, 256, 64), (1, 1, 1, 128, 64)])
@pytest.mark.parametrize("ids", ["runs", "unsorted", "gapped"])
def test_host_builder_bit_exact(si, shape, ids):
    """runs: packed documents with consecutive ids; unsorted: independent random ids;
    gapped: sorted runs whose ids skip values (ranges overlap without a shared id)."""
    B, Lq, Lkv, BQ, BK = shape
    spec = dict(SPECS[si])
    if not spec.get("doc") and ids != "runs":
        pytest.skip("ids only matter with the document mask")
    if spec.get("doc"):
        w = random_case(2000 + si, B=B, Lq=Lq, Lkv=Lkv, D=8, doc=True, n_docs=9, doc_sorted=ids != "unsorted")
        spec["q_doc"], spec["kv_doc"] = w.q_doc, w.kv_doc
        if ids == "gapped":
            spec["q_doc"] = (w.q_doc * 2).astype(np.int32)
            spec["kv_doc"] = (w.kv_doc * 2 + (1 if Lq != Lkv else 0)).astype(np.int32)
    got = build_host(spec, B, Lq, Lkv, BQ, BK)
    ref = ref_bm.block_mask(spec, B, Lq, Lkv, BQ, BK)
    for k in KEYS:
        assert np.array_equal(got[k], ref[k]), k


def test_host_builder_causal_closed_form_counts():
    """Causal at T = 8192 with 128-blocks: 2016 full, 64 partial tiles (the page's ~50% skipped)."""
    got = build_host({"causal": True}, 1, 8192, 8192, 128, 128)
    assert got["full_kv_num_blocks"].sum() == 2016 and got["kv_num_blocks"].sum() == 64


def test_host_builder_empty_and_errors():
    fa = _fa()
    bm = fa.flexattn_block_mask_build_host(fa.FA_MASK_CAUSAL, 1, 70, 0, 128, 64)
    assert bm.kv_num_blocks.numpy().tolist() == [[[0]]] and bm.full_kv_num_blocks.numpy().tolist() == [[[0]]]
    with pytest.raises(fa.FlexAttnError) as e:
        fa.flexattn_block_mask_build_host(fa.FA_MASK_CAUSAL | fa.FA_MASK_PREFIX_LM, 1, 64, 64, 64, 64, prefix_len=3)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    with pytest.raises(fa.FlexAttnError) as e:
        fa.flexattn_block_mask_build_host(fa.FA_MASK_NONE, 1, 64, 64, 96, 64)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FlexAttnError) as e:
        fa.flexattn_block_mask_build_host(fa.FA_MASK_DOC, 1, 64, 64, 64, 64)
    assert e.value.status == fa.FA_ERR_INVALID_ARG


def _expected_order(full_num, part_num):
    """The documented schedule: per row set, query blocks by decreasing 4 * full + 5 * partial
    live tiles, ties by increasing query block."""
    Bm, Hm, nqb = full_num.shape
    out = np.empty_like(full_num)
    for bm in range(Bm):
        for hm in range(Hm):
            cost = 4 * full_num[bm, hm].astype(np.int64) + 5 * part_num[bm, hm].astype(np.int64)
            out[bm, hm] = sorted(range(nqb), key=lambda qb: (-cost[qb], qb))
    return out


@pytest.mark.parametrize("si", range(len(SPECS)))
@pytest.mark.parametrize("shape", [(2, 333, 333, 128, 128), (1, 700, 517, 64, 128), (2, 2000, 2000, 128, 64),
                                   (1, 1, 1, 128, 64)])
def test_host_row_order(si, shape):
    """The optional schedule array: a permutation of the query blocks of each row set in the
    documented cost order; the mask arrays are the same with and without it."""
    B, Lq, Lkv, BQ, BK = shape
    spec = dict(SPECS[si])
    if spec.get("doc"):
        w = random_case(3000 + si, B=B, Lq=Lq, Lkv=Lkv, D=8, doc=True, n_docs=7)
        spec["q_doc"], spec["kv_doc"] = w.q_doc, w.kv_doc
    fa = _fa()
    qd = kd = None
    if spec.get("doc"):
        qd = np.ascontiguousarray(spec["q_doc"], np.int32)
        kd = np.ascontiguousarray(spec["kv_doc"], np.int32)
    kw = dict(q_doc=qd, kv_doc=kd, window=spec.get("window") or 0, prefix_len=spec.get("prefix_len") or 0)
    bm = fa.flexattn_block_mask_build_host(_mask_kind(fa, spec), B, Lq, Lkv, BQ, BK, row_order=True, **kw)
    plain = fa.flexattn_block_mask_build_host(_mask_kind(fa, spec), B, Lq, Lkv, BQ, BK, **kw)
    for k in KEYS:
        assert np.array_equal(getattr(bm, k).numpy(), getattr(plain, k).numpy()), k
    order = bm.row_order.numpy()
    want = _expected_order(bm.full_kv_num_blocks.numpy(), bm.kv_num_blocks.numpy())
    assert np.array_equal(order, want)
    for row in order.reshape(-1, order.shape[-1]):
        assert np.array_equal(np.sort(row), np.arange(order.shape[-1]))


def test_host_row_order_identity_beyond_limit():
    """More than 8192 query blocks in a row set: the schedule is the identity order."""
    fa = _fa()
    nqb = 8193
    bm = fa.flexattn_block_mask_build_host(fa.FA_MASK_CAUSAL, 1, nqb * 64, 64, 64, 64, row_order=True)
    assert np.array_equal(bm.row_order.numpy()[0, 0], np.arange(nqb))
    small = fa.flexattn_block_mask_build_host(fa.FA_MASK_CAUSAL, 1, 8192 * 64, 8192 * 64 // 4, 64, 64,
                                              row_order=True)
    want = _expected_order(small.full_kv_num_blocks.numpy(), small.kv_num_blocks.numpy())
    assert np.array_equal(small.row_order.numpy(), want)
    # Row 2047 (2047 full + 1 partial) costs most; rows past the keys tie (2048 full each) and
    # follow in increasing order; row 0 (one partial tile) is last.
    o = want[0, 0]
    assert list(o[:4]) == [2047, 2048, 2049, 2050] and o[-1] == 0

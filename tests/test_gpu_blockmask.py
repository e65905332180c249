"""GPU: the device BlockMask builder is bit-exact with the exhaustive oracle."""
import numpy as np
import pytest

from oracle import blockmask as ref_bm
from workloads import make_workload, random_case

pytestmark = pytest.mark.gpu

KEYS = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices")


def _dev():
    import torch
    return torch.device("cuda", 0)


def _mask_kind(fa, spec):
    m = 0
    m |= fa.FA_MASK_DOC if spec.get("doc") else 0
    m |= fa.FA_MASK_CAUSAL if spec.get("causal") else 0
    m |= fa.FA_MASK_WINDOW if spec.get("window") is not None else 0
    m |= fa.FA_MASK_PREFIX_LM if spec.get("prefix_len") is not None else 0
    return m


def build_gpu(spec, B, Lq, Lkv, BQ, BK):
    import torch
    import block_sparse_masked_blockmask_amd as fa
    dev = _dev()
    qd = kd = None
    if spec.get("doc"):
        qd = torch.from_numpy(np.ascontiguousarray(spec["q_doc"], np.int32)).to(dev)
        # One id array for both sides (the builder's self-attention closed form) when the
        # spec's ids are one array; separate copies otherwise.
        kd = qd if spec["kv_doc"] is spec["q_doc"] else \
            torch.from_numpy(np.ascontiguousarray(spec["kv_doc"], np.int32)).to(dev)
    bm = fa.flexattn_block_mask_build(_mask_kind(fa, spec), B, Lq, Lkv, BQ, BK, q_doc=qd, kv_doc=kd,
                                      window=spec.get("window") or 0, prefix_len=spec.get("prefix_len") or 0,
                                      device=dev)
    torch.cuda.synchronize()
    return {k: getattr(bm, k).cpu().numpy() for k in KEYS}


def assert_same(got, ref, rows=None):
    if rows is None:
        for k in KEYS:
            assert np.array_equal(got[k], ref[k]), k
    else:
        for bm, qb in rows:
            for k in KEYS:
                assert np.array_equal(got[k][bm, 0, qb], ref[k][bm, 0, qb]), (k, bm, qb)


SPECS = [
    {}, {"causal": True}, {"window": 37}, {"causal": True, "window": 100}, {"prefix_len": 77},
    {"prefix_len": 50, "window": 90}, {"doc": True}, {"doc": True, "causal": True},
    {"doc": True, "causal": True, "window": 64}, {"doc": True, "prefix_len": 30},
]


@pytest.mark.parametrize("si", range(len(SPECS)))
@pytest.mark.parametrize("shape", [(2, 333, 333, 128, 128), (1, 700, 517, 64, 128), (2, 260, 390, 128, 64), (1, 64, 64, 64, 64),
                                   (2, 600, 600, 256, 64), (1, 300, 700, 256, 128)])
@pytest.mark.parametrize("ids", ["runs", "unsorted", "gapped"])
def test_random_cases_bit_exact(si, shape, ids):
    """runs: packed documents with consecutive ids; unsorted: independent random ids;
    gapped: sorted runs whose ids skip values (ranges overlap without a shared id)."""
    B, Lq, Lkv, BQ, BK = shape
    spec = dict(SPECS[si])
    if not spec.get("doc") and ids != "runs":
        pytest.skip("ids only matter with the document mask")
    if spec.get("doc"):
        w = random_case(1000 + si, B=B, Lq=Lq, Lkv=Lkv, D=8, doc=True, n_docs=9, doc_sorted=ids != "unsorted")
        spec["q_doc"], spec["kv_doc"] = w.q_doc, w.kv_doc
        if ids == "gapped":
            spec["q_doc"] = (w.q_doc * 2).astype(np.int32)
            spec["kv_doc"] = (w.kv_doc * 2 + (1 if Lq != Lkv else 0)).astype(np.int32)
    got = build_gpu(spec, B, Lq, Lkv, BQ, BK)
    ref = ref_bm.block_mask(spec, B, Lq, Lkv, BQ, BK)
    assert_same(got, ref)


def test_empty_lengths():
    got = build_gpu({"causal": True}, 1, 0, 100, 128, 128)
    assert got["kv_num_blocks"].size == 0
    got = build_gpu({"doc": True, "q_doc": np.zeros((1, 100), np.int32), "kv_doc": np.zeros((1, 1), np.int32)[:, :0]},
                    1, 100, 0, 128, 128)
    assert got["kv_num_blocks"].tolist() == [[[0]]] and got["full_kv_num_blocks"].tolist() == [[[0]]]


def _spec_of(w):
    return dict(doc=w.doc, causal=w.causal, window=w.window, prefix_len=w.prefix_len, q_doc=w.q_doc, kv_doc=w.kv_doc)


@pytest.mark.parametrize("name,bq,bk", [
    ("grouped_variate_4x17_f32", 128, 128),
    ("grouped_variate_4096g_bf16", 128, 128),
    ("grouped_variate_4096g_bf16", 256, 64),
    ("doc_causal_b4h16t8192_bf16", 256, 64),
    ("swa1024_gqa32x8_softcap50_t16384_bf16", 256, 64),
    ("doc_causal_b4h16t8192_bf16", 128, 128),
    ("swa1024_gqa32x8_softcap50_t16384_bf16", 128, 128),
    ("dense_b1h32s24576_bf16", 128, 128),
])
def test_workload_block_masks(name, bq, bk):
    w = make_workload(name, with_tensors=False)
    spec = _spec_of(w)
    got = build_gpu(spec, w.B, w.Lq, w.Lkv, bq, bk)
    nqb = -(-w.Lq // bq)
    Bm = w.B if w.doc else 1
    if name.startswith("grouped_variate_4096g"):
        # Exhaustive rows: every 16th query block, the first and the last.
        rows = [(0, qb) for qb in sorted(set(range(0, nqb, 16)) | {nqb - 1})]
    else:
        rows = [(b, qb) for b in range(Bm) for qb in range(nqb)]
    ref = ref_bm.block_mask(spec, w.B, w.Lq, w.Lkv, bq, bk, rows=rows)
    assert_same(got, ref, rows)
    if name == "swa1024_gqa32x8_softcap50_t16384_bf16" and (bq, bk) == (128, 128):
        assert (int(got["full_kv_num_blocks"].sum()), int(got["kv_num_blocks"].sum())) == (868, 248)
    if name == "grouped_variate_4096g_bf16" and bk == 128:
        # Every row of the packed groups has only partial tiles (no group is tile-aligned).
        tot_p = int(got["kv_num_blocks"].sum())
        print(f"{name}: partial tiles {tot_p}, full {int(got['full_kv_num_blocks'].sum())}")


@pytest.mark.parametrize("mask", ["doc_sorted", "doc_unsorted", "causal_window"])
def test_multi_pass_rows(mask):
    """Rows longer than one classification pass (9,375 kv blocks of 64 keys, three passes):
    the device lists equal the oracle on sampled rows and the host builder on every row."""
    import block_sparse_masked_blockmask_amd as fa
    rng = np.random.default_rng(77)
    B, Lq, Lkv, BQ, BK = 1, 700, 600_000, 128, 64
    if mask == "causal_window":
        spec = {"causal": True, "window": 250_000}
        Lq = Lkv = 600_000
    else:
        qd = np.sort(rng.integers(0, 40, size=(B, Lq))).astype(np.int32)
        kd = np.sort(rng.integers(0, 40, size=(B, Lkv))).astype(np.int32)
        if mask == "doc_unsorted":
            # ids repeat far apart: tiles the closed forms cannot settle in every pass
            kd = (np.arange(Lkv, dtype=np.int64) // 5000 % 40).astype(np.int32)[None, :]
        spec = {"doc": True, "q_doc": qd, "kv_doc": kd}
    got = build_gpu(spec, B, Lq, Lkv, BQ, BK)
    nqb = -(-Lq // BQ)
    rows = [(0, qb) for qb in sorted({0, nqb // 2, nqb - 1})]
    ref = ref_bm.block_mask(spec, B, Lq, Lkv, BQ, BK, rows=rows)
    assert_same(got, ref, rows)
    host = fa.flexattn_block_mask_build_host(
        _mask_kind(fa, spec), B, Lq, Lkv, BQ, BK,
        q_doc=None if mask == "causal_window" else np.ascontiguousarray(spec["q_doc"]),
        kv_doc=None if mask == "causal_window" else np.ascontiguousarray(spec["kv_doc"]),
        window=spec.get("window") or 0)
    for k in KEYS:
        assert np.array_equal(got[k], getattr(host, k).numpy()), k


@pytest.mark.parametrize("alias", [True, False])
def test_aliased_ids_equal_copies(alias):
    """The same ids passed as one array (self-attention closed form for diagonal tiles) or as
    two copies give identical lists, equal to the oracle."""
    w = random_case(2100, B=2, Lq=3000, Lkv=3000, D=8, doc=True, n_docs=25)
    spec = {"doc": True, "causal": True, "q_doc": w.q_doc, "kv_doc": w.q_doc if alias else w.q_doc.copy()}
    got = build_gpu(spec, 2, 3000, 3000, 128, 64)
    ref = ref_bm.block_mask(spec, 2, 3000, 3000, 128, 64)
    assert_same(got, ref)

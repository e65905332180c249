"""Pins of the BlockMask reference: brute force per tile, closed-form counts,
and the page's skip ratios (tests/golden/page_skip_ratios.json)."""
import json
import os

import numpy as np
import pytest

from oracle import blockmask as BM
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_lists(bm, spec, B, Lq, Lkv, BQ, BK):
    Bm, Hm, nqb, nkvb = BM.dims(spec, B, Lq, Lkv, BQ, BK)
    for b in range(Bm):
        for qb in range(nqb):
            cls = [brute.block_class(b, qb, kb, Lq, Lkv, BQ, BK, spec) for kb in range(nkvb)]
            part = [kb for kb, c in enumerate(cls) if c == "partial"]
            full = [kb for kb, c in enumerate(cls) if c == "full"]
            assert bm["kv_num_blocks"][b, 0, qb] == len(part)
            assert bm["full_kv_num_blocks"][b, 0, qb] == len(full)
            assert list(bm["kv_indices"][b, 0, qb, :len(part)]) == part
            assert list(bm["full_kv_indices"][b, 0, qb, :len(full)]) == full
            assert not bm["kv_indices"][b, 0, qb, len(part):].any()
            assert not bm["full_kv_indices"][b, 0, qb, len(full):].any()


CASES = [
    ({}, 1, 13, 13, 4, 4),
    ({"causal": True}, 1, 17, 17, 4, 4),
    ({"causal": True}, 1, 16, 21, 4, 8),
    ({"causal": True, "window": 5}, 1, 30, 30, 4, 4),
    ({"window": 3}, 1, 19, 19, 8, 4),
    ({"prefix_len": 6}, 1, 25, 25, 4, 4),
    ({"prefix_len": 6, "window": 7}, 1, 25, 25, 4, 4),
    ({"doc": True}, 2, 27, 27, 4, 4),
    ({"doc": True, "causal": True}, 2, 27, 27, 8, 4),
    ({"doc": True, "causal": True, "window": 6}, 2, 33, 29, 4, 4),
    ({"doc": True, "prefix_len": 5}, 2, 21, 21, 4, 8),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_block_mask_matches_per_tile_brute_force(ci):
    spec, B, Lq, Lkv, BQ, BK = CASES[ci]
    spec = dict(spec)
    if spec.get("doc"):
        r = np.random.default_rng(ci)
        # Sorted runs for batch 0, unsorted ids for batch 1.
        a = np.sort(r.integers(0, 5, Lq)).astype(np.int32)
        bq = r.integers(0, 4, Lq).astype(np.int32)
        spec["q_doc"] = np.stack([a, bq])
        a2 = np.sort(r.integers(0, 5, Lkv)).astype(np.int32)
        bk = r.integers(0, 4, Lkv).astype(np.int32)
        spec["kv_doc"] = np.stack([a2, bk])
    bm = BM.block_mask(spec, B, Lq, Lkv, BQ, BK)
    _check_lists(bm, spec, B, Lq, Lkv, BQ, BK)


def test_causal_closed_form():
    # n x n tiles with BQ | T: strictly-lower tiles full, diagonal partial, rest empty.
    for T, Bt in [(8192, 128), (1024, 64), (512, 128)]:
        n = T // Bt
        full, part = BM.tile_counts(BM.block_mask({"causal": True}, 1, T, T, Bt, Bt))
        assert (full, part) == (n * (n - 1) // 2, n)


def test_causal_window_closed_form():
    # W = m * B: row r has full tiles kb in [r-m+1, r-1] and partial tiles at
    # kb = r (the diagonal) and, once r >= m, at kb = r - m (the window edge).
    for T, W, Bt in [(16384, 1024, 128), (8192, 1024, 128), (4096, 512, 64)]:
        n, m = T // Bt, W // Bt
        full, part = BM.tile_counts(BM.block_mask({"causal": True, "window": W}, 1, T, T, Bt, Bt))
        exp_full = sum(min(r, m - 1) for r in range(n))
        exp_part = sum(1 + (r >= m) for r in range(n))
        assert (full, part) == (exp_full, exp_part)
    full, part = BM.tile_counts(BM.block_mask({"causal": True, "window": 1024}, 1, 16384, 16384))
    assert (full, part) == (868, 248)


def test_page_skip_ratios():
    g = json.load(open(os.path.join(GOLDEN, "page_skip_ratios.json")))
    t = g["tile"]
    c = g["causal"]
    full, part = BM.tile_counts(BM.block_mask({"causal": True}, 1, c["T"], c["T"], t, t))
    n = (c["T"] // t) ** 2
    skipped = 1 - (full + part) / n
    assert abs(skipped - c["skipped_fraction_approx"]) <= c["tolerance"]
    w = g["sliding_window_causal"]
    full, part = BM.tile_counts(BM.block_mask({"causal": True, "window": w["W"]}, 1, w["T"], w["T"], t, t))
    n = (w["T"] // t) ** 2
    assert 1 - (full + part) / n > w["skipped_fraction_min"]


def test_aligned_groups_give_full_diagonal():
    ids = np.repeat(np.arange(6), 64).astype(np.int32)[None]   # groups of 64, tiles of 64
    bm = BM.block_mask({"doc": True, "q_doc": ids, "kv_doc": ids}, 1, 384, 384, 64, 64)
    assert BM.tile_counts(bm) == (6, 0)
    assert list(bm["full_kv_indices"][0, 0, :, 0]) == list(range(6))


def test_no_mask_ragged_all_full():
    bm = BM.block_mask({}, 1, 300, 200, 128, 128)
    assert BM.tile_counts(bm) == (3 * 2, 0)


def test_sampled_rows_equal_full_build():
    r = np.random.default_rng(3)
    ids = np.sort(r.integers(0, 30, 1000)).astype(np.int32)[None]
    spec = {"doc": True, "causal": True, "q_doc": ids, "kv_doc": ids}
    full = BM.block_mask(spec, 1, 1000, 1000, 64, 64)
    part = BM.block_mask(spec, 1, 1000, 1000, 64, 64, rows=[(0, 3), (0, 15)])
    for qb in (3, 15):
        for key in full:
            assert np.array_equal(full[key][0, 0, qb], part[key][0, 0, qb])

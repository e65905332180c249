"""BlockMask reference by exhaustive evaluation — TEST INFRASTRUCTURE.

FlexAttention guide, "Systems Mechanics", item 1 (128x128 tile block sparsity):
the mask predicate is evaluated over each tile's bounding box; a tile whose
pairs are all allowed is full (computed without mask branches), one with none
allowed is empty (never loaded), anything else is partial (token-level mask).

Layout of the result (field names of FlexAttention's BlockMask; the order and
padding are this project's reading, the pages give none):
  kv_num_blocks[Bm][Hm][nQB]          number of partial tiles in the row,
  kv_indices[Bm][Hm][nQB][nKVB]       their kv-block indices, ascending,
  full_kv_num_blocks[Bm][Hm][nQB]     number of full tiles,
  full_kv_indices[Bm][Hm][nQB][nKVB]  their indices, ascending;
unused list entries are 0. Bm = B when the document predicate is on (it depends
on b), else 1; Hm = 1 (no predicate here depends on the head).
Ragged edges: only in-range pairs are evaluated; a ragged tile whose in-range
pairs are all allowed counts as full.
"""
from __future__ import annotations

import numpy as np

from .attention import mask_mod


def _row_classes(spec, b, qb, Lq, Lkv, BQ, BK):
    """Classes of every kv tile of one q-block row: 2 = full, 1 = partial, 0 = empty."""
    q0, q1 = qb * BQ, min(Lq, (qb + 1) * BQ)
    keep = mask_mod(np.arange(q0, q1), np.arange(Lkv),
                    q_doc_row=None if spec.get("q_doc") is None else spec["q_doc"][b],
                    kv_doc_row=None if spec.get("kv_doc") is None else spec["kv_doc"][b],
                    doc=spec.get("doc", False), causal=spec.get("causal", False),
                    window=spec.get("window"), prefix_len=spec.get("prefix_len"))
    nkvb = -(-Lkv // BK)
    pad = nkvb * BK - Lkv
    # Pad out-of-range columns so that they count as allowed for "all" and not for "any".
    k_all = np.concatenate([keep, np.ones((keep.shape[0], pad), bool)], axis=1)
    k_any = np.concatenate([keep, np.zeros((keep.shape[0], pad), bool)], axis=1)
    all_ = k_all.reshape(keep.shape[0], nkvb, BK).all(axis=(0, 2))
    any_ = k_any.reshape(keep.shape[0], nkvb, BK).any(axis=(0, 2))
    cls = np.where(all_, 2, np.where(any_, 1, 0))
    return cls


def dims(spec, B, Lq, Lkv, BQ, BK):
    Bm = B if spec.get("doc") else 1
    return Bm, 1, -(-Lq // BQ), -(-Lkv // BK)


def block_mask(spec, B, Lq, Lkv, BQ=128, BK=128, rows=None):
    """Exhaustive BlockMask. rows: optional list of (bm, qb) to fill (others left 0).

    Returns a dict of int32 arrays with the layout described in the module doc.
    """
    Bm, Hm, nqb, nkvb = dims(spec, B, Lq, Lkv, BQ, BK)
    out = {
        "kv_num_blocks": np.zeros((Bm, Hm, nqb), np.int32),
        "kv_indices": np.zeros((Bm, Hm, nqb, nkvb), np.int32),
        "full_kv_num_blocks": np.zeros((Bm, Hm, nqb), np.int32),
        "full_kv_indices": np.zeros((Bm, Hm, nqb, nkvb), np.int32),
    }
    todo = rows if rows is not None else [(bm, qb) for bm in range(Bm) for qb in range(nqb)]
    for bm, qb in todo:
        cls = _row_classes(spec, bm, qb, Lq, Lkv, BQ, BK)
        part = np.flatnonzero(cls == 1)
        full = np.flatnonzero(cls == 2)
        out["kv_num_blocks"][bm, 0, qb] = len(part)
        out["kv_indices"][bm, 0, qb, :len(part)] = part
        out["full_kv_num_blocks"][bm, 0, qb] = len(full)
        out["full_kv_indices"][bm, 0, qb, :len(full)] = full
    return out


def tile_counts(bm_dict):
    """(full, partial) tile totals over all rows."""
    return int(bm_dict["full_kv_num_blocks"].sum()), int(bm_dict["kv_num_blocks"].sum())


def transposed_block_mask(spec, B, Lq, Lkv, BQ=128, BK=128):
    """The column view of the same tile classes, for a backward that walks kv blocks.

    For each mask row bm and kv block kb: the q blocks whose (qb, kb) tile is
    partial (q_indices) or full (full_q_indices), ascending, with their counts;
    unused entries 0. Shapes: q_num_blocks / full_q_num_blocks [Bm][Hm][nKVB],
    q_indices / full_q_indices [Bm][Hm][nKVB][nQB]. (The pages give no layout;
    the field names follow FlexAttention's BlockMask, whose backward needs this
    view of the tiles.)
    """
    Bm, Hm, nqb, nkvb = dims(spec, B, Lq, Lkv, BQ, BK)
    cls = np.zeros((Bm, nqb, nkvb), np.int32)
    for bm in range(Bm):
        for qb in range(nqb):
            cls[bm, qb] = _row_classes(spec, bm, qb, Lq, Lkv, BQ, BK)
    out = {
        "q_num_blocks": np.zeros((Bm, Hm, nkvb), np.int32),
        "q_indices": np.zeros((Bm, Hm, nkvb, nqb), np.int32),
        "full_q_num_blocks": np.zeros((Bm, Hm, nkvb), np.int32),
        "full_q_indices": np.zeros((Bm, Hm, nkvb, nqb), np.int32),
    }
    for bm in range(Bm):
        for kb in range(nkvb):
            part = np.flatnonzero(cls[bm, :, kb] == 1)
            full = np.flatnonzero(cls[bm, :, kb] == 2)
            out["q_num_blocks"][bm, 0, kb] = len(part)
            out["q_indices"][bm, 0, kb, :len(part)] = part
            out["full_q_num_blocks"][bm, 0, kb] = len(full)
            out["full_q_indices"][bm, 0, kb, :len(full)] = full
    return out

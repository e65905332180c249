// Tile classification shared by the device BlockMask builder and the host builder.
//
// FlexAttention guide, "Systems Mechanics", item 1: the mask predicate is evaluated over each
// tile's bounding box; all-true tiles are full, all-false tiles are empty, the rest partial.
// Here the box is the tile's in-range pairs. The closed forms below settle a tile from its
// corners and from per-block document-id summaries; the tiles they cannot settle are evaluated
// pair by pair with mask_pair.
#pragma once
#include <hip/hip_runtime.h>

#include "flexattn.h"

namespace fa {

// mask_mod for one (query, key) pair: the AND of the enabled predicates on absolute positions
// (causal and window from the guide's "Implementation" demo, the document and prefix-LM masks
// from "Production Engineering").
__host__ __device__ inline bool mask_pair_flags(int flags, int window, int prefix_len, int i, int j, int qdoc,
                                                int kvdoc) {
  bool keep = true;
  if (flags & FA_MASK_DOC) keep = keep && (qdoc == kvdoc);
  if (flags & FA_MASK_CAUSAL) keep = keep && (i >= j);
  if (flags & FA_MASK_WINDOW) keep = keep && (i - j < window);
  if (flags & FA_MASK_PREFIX_LM) keep = keep && ((j < prefix_len) || (i >= j));
  return keep;
}

// Class of the tile [q0, q1) x [k0, k1) (non-empty ranges): 0 empty, 1 partial, 2 full, 3 not
// settled by closed forms. Under DOC, [qmin, qmax] and [kmin, kmax] are the id ranges of the
// query and key blocks, and qdense / kdense flag blocks whose consecutive ids differ by 0 or 1
// (every id of the range then occurs in the block). self_ids: the query and key document ids
// are one array (same memory, q_len == kv_len), so position i has the same id on both sides.
__host__ __device__ inline int classify_closed(int flags, int window, int prefix_len, int q0, int q1, int k0, int k1,
                                               int qmin, int qmax, int qdense, int kmin, int kmax, int kdense,
                                               bool self_ids = false) {
  const int dmin = q0 - (k1 - 1), dmax = (q1 - 1) - k0;  // range of q - kv over the box
  bool all = true, none = false;
  if (flags & FA_MASK_CAUSAL) {
    all = all && dmin >= 0;
    none = none || dmax < 0;
  }
  if (flags & FA_MASK_WINDOW) {
    all = all && dmax < window;
    none = none || dmin >= window;
  }
  if (flags & FA_MASK_PREFIX_LM) {
    all = all && ((k1 - 1 < prefix_len) || dmin >= 0);
    none = none || (k0 >= prefix_len && dmax < 0);
  }
  const bool index_all = all;
  if (flags & FA_MASK_DOC) {
    all = all && (qmin == qmax && kmin == kmax && qmin == kmin);
    none = none || (qmax < kmin || kmax < qmin);
  }
  if (all) return 2;
  if (none) return 0;
  // A box that holds a diagonal pair (i, i) has an allowed pair: causal, window (> 0) and
  // prefix-LM all allow j = i, and with self_ids so does the document predicate.
  const bool diag = (q0 > k0 ? q0 : k0) < (q1 < k1 ? q1 : k1);
  if (diag && (self_ids || !(flags & FA_MASK_DOC))) return 1;
  if (!(flags & FA_MASK_DOC)) {
    // Causal and window together allow exactly the pairs with q - kv in [0, window): the box's
    // q - kv values form one integer interval, and each predicate alone was not all-false, so
    // the interval meets [0, window) and some pair is allowed. Prefix-LM alone is one
    // predicate that is not all-false.
    if (!(flags & FA_MASK_PREFIX_LM)) return 1;
    if (!(flags & FA_MASK_WINDOW)) return 1;
    return 3;
  }
  // Document ids with every index predicate true on the whole box: the tile is non-empty iff
  // the blocks share an id, which dense blocks with overlapping ranges do.
  if (index_all && qdense && kdense) return 1;
  return 3;
}

// BlockMask counts and list entries come from caller memory. Kernels that walk the lists clamp
// each count into [0, cap] (cap = the list length) and replace an entry outside [0, n) by n, a
// block past the last one, which every walker skips (its rows lie beyond the sequence), so that a
// corrupt BlockMask cannot send a kernel outside its arrays.
__host__ __device__ inline int clamp_count(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }
__host__ __device__ inline int sanitize_block(int x, int n) { return (x >= 0 && x < n) ? x : n; }

// Schedule key of a BlockMask row (the optional row_order of fa_block_mask): rows are sorted by
// increasing key, i.e. by decreasing estimated cost 4 * full + 5 * partial live tiles (a partial
// tile also evaluates the mask on every score), ties by increasing query block. The cost is
// saturated to 19 bits and the query block takes the low 13 bits, so keys are unique and an
// ascending sort of them is the whole order.
constexpr int kRowOrderMax = 8192;  // query blocks per row set that are sorted (else identity)
constexpr unsigned kRowOrderQbMask = kRowOrderMax - 1;
__host__ __device__ inline unsigned row_order_key(int nfull, int npart, int qb) {
  const unsigned cmax = (1u << 19) - 1;
  unsigned cost = 4u * (unsigned)nfull + 5u * (unsigned)npart;
  cost = cost < cmax ? cost : cmax;
  return ((cmax - cost) << 13) | (unsigned)qb;
}

}  // namespace fa

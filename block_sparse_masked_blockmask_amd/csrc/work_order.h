// Work order and key intervals shared by the bf16 forward kernels (fwd.hip, fwd_pipe.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <climits>

#include "device_common.h"
#include "launch.h"

namespace fa {

struct WorkItem {
  int b, hq, hkv, qb, split;
};

// MODE 0: plain forward; 1: split-KV; 2: split-KV with the query heads of one kv head packed
// into one workgroup (rows = (head, query) pairs, all queries of all heads of the group).
// wg: the work item's index in dispatch order (the workgroup id, or the workgroup id / 4 for the
// split-key fp32 kernel, whose four workgroups share one work item).
template <int MODE = 0>
__device__ __forceinline__ WorkItem decode_work(const FwdArgs& a, int wg) {
  int w = xcd_remap(wg, a.total_wg);
  // Order: splits of one work item fastest (they read the same Q rows), then query heads of
  // one kv head (they read the same K/V tiles), then query blocks from the last (most tiles
  // under causal masks) to the first, then kv head, batch.
  WorkItem it;
  it.split = 0;
  if constexpr (MODE == 0) {
    if (a.row_order != nullptr) {
      // Scheduled order: rank r of the row order outermost, so the costliest query blocks of
      // every (batch, head) start first, and consecutive workgroups (which the hardware deals
      // round-robin to the 8 XCDs) take the (batch, kv head) pairs fastest, then the query heads
      // of a kv head: with 8 | B * Hkv, XCD x always serves pairs x, x + 8, ..., so each K/V
      // head is read through one L2.
      const int w0 = wg;
      const int npair = a.B * a.Hkv;
      const int per_rank = npair * a.group;
      const int idx = w0 % per_rank, r = w0 / per_rank;
      const int pair = idx % npair, g = idx / npair;
      it.hkv = pair % a.Hkv;
      it.b = pair / a.Hkv;
      it.hq = it.hkv * a.group + g;
      const int bm = a.Bm == 1 ? 0 : it.b;
      const int hm = a.Hm == 1 ? 0 : it.hq;
      it.qb = min(max(a.row_order[((int64_t)bm * a.Hm + hm) * a.nqb + r], 0), a.nqb - 1);
      return it;
    }
  }
  if constexpr (MODE > 0) {
    it.split = w % a.nsplit;
    w /= a.nsplit;
  }
  int g = 0;
  if constexpr (MODE != 2) {
    g = w % a.group;
    w /= a.group;
  }
  const int qbr = w % a.nqb;
  w /= a.nqb;
  // w now indexes the (batch, kv head) pairs in dispatch order. The contiguous ranges that the
  // XCDs receive are taken over a permutation of the pairs: range c holds pairs c, c + 8,
  // c + 16, ..., so every XCD mixes batches (whose document structures, and therefore work,
  // differ) instead of taking one batch's heads. All query blocks of a pair stay in one range.
  const int npair = a.B * a.Hkv;
  const int q8 = npair / 8, r8 = npair % 8;
  int c, k;
  if (w < r8 * (q8 + 1)) {
    c = w / (q8 + 1);
    k = w % (q8 + 1);
  } else {
    c = r8 + (w - r8 * (q8 + 1)) / q8;
    k = (w - r8 * (q8 + 1)) % q8;
  }
  const int pair = 8 * k + c;
  it.hkv = pair % a.Hkv;
  it.b = pair / a.Hkv;
  it.qb = a.nqb - 1 - qbr;
  it.hq = it.hkv * a.group + g;
  return it;
}

// Allowed key interval [lo, hi) of query qi under the index predicates and the key count.
// Causal, window and prefix-LM together allow exactly one interval: causal gives hi = i + 1,
// prefix-LM hi = max(prefix_len, i + 1), window lo = i - window + 1; the key count bounds hi.
__device__ __forceinline__ void key_interval(const FwdArgs& a, int qi, int& lo, int& hi) {
  lo = INT_MIN / 2;
  hi = a.Lkv;
  if (a.flags & FA_MASK_CAUSAL) hi = min(hi, qi + 1);
  if (a.flags & FA_MASK_PREFIX_LM) hi = min(hi, max(a.prefix_len, qi + 1));
  if (a.flags & FA_MASK_WINDOW) lo = qi - a.window + 1;
  hi = max(hi, lo);
}

}  // namespace fa

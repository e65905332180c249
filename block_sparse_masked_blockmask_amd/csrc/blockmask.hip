// BlockMask construction on the device (gfx950).
//
// FlexAttention guide, "Systems Mechanics", item 1: the mask predicate is evaluated over each
// tile's bounding box; all-true tiles are full, all-false tiles are empty (never visited), the
// rest are partial. Here the box is the tile's in-range pairs. Each (mask row, query block) row
// is classified by one workgroup:
//   1. closed forms decide most tiles exactly: the index predicates (causal, window, prefix-LM)
//      are monotone in q - kv or kv, so their all-true / all-false conditions are corner tests;
//      document ids use per-block [min, max] ranges (equal single ids: full; disjoint: empty);
//   2. tiles that the closed forms cannot settle are evaluated pair by pair by the whole
//      workgroup (exact for any ids, sorted or not);
//   3. a block-wide ballot scan writes the full and partial lists in ascending kv order and
//      zero-fills their tails.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace fa {

__global__ __launch_bounds__(256) void bm_summaries(BlockMaskArgs a) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int nq = a.B * a.nqb, nk = a.B * a.nkvb;
  const int* ids;
  int lo, hi;
  int* dst;
  if (t < nq) {
    const int b = t / a.nqb, blk = t % a.nqb;
    ids = a.q_doc + (int64_t)b * a.Lq;
    lo = blk * a.BQ;
    hi = min(a.Lq, lo + a.BQ);
    dst = a.qsum + 2 * t;
  } else if (t < nq + nk) {
    const int u = t - nq;
    const int b = u / a.nkvb, blk = u % a.nkvb;
    ids = a.kv_doc + (int64_t)b * a.Lkv;
    lo = blk * a.BK;
    hi = min(a.Lkv, lo + a.BK);
    dst = a.kvsum + 2 * u;
  } else {
    return;
  }
  int mn = ids[lo], mx = ids[lo];
  for (int i = lo + 1; i < hi; ++i) {
    const int d = ids[i];
    mn = min(mn, d);
    mx = max(mx, d);
  }
  dst[0] = mn;
  dst[1] = mx;
}

// Class codes: 0 empty, 1 partial, 2 full, 3 undecided by closed forms.
__device__ __forceinline__ int classify_closed(const BlockMaskArgs& a, int q0, int q1, int k0, int k1,
                                               int qmin, int qmax, int kmin, int kmax) {
  const int dmin = q0 - (k1 - 1), dmax = (q1 - 1) - k0;  // range of q - kv over the box
  bool all = true, none = false;
  if (a.flags & FA_MASK_CAUSAL) {
    all = all && dmin >= 0;
    none = none || dmax < 0;
  }
  if (a.flags & FA_MASK_WINDOW) {
    all = all && dmax < a.window;
    none = none || dmin >= a.window;
  }
  if (a.flags & FA_MASK_PREFIX_LM) {
    all = all && ((k1 - 1 < a.prefix_len) || dmin >= 0);
    none = none || (k0 >= a.prefix_len && dmax < 0);
  }
  if (a.flags & FA_MASK_DOC) {
    all = all && (qmin == qmax && kmin == kmax && qmin == kmin);
    none = none || (qmax < kmin || kmax < qmin);
  }
  if (all) return 2;
  if (none) return 0;
  // Without document ids, causal and window together allow exactly the pairs with q - kv in
  // [0, window): the box's q - kv values form one integer interval, and each predicate alone
  // was not all-false, so the interval meets [0, window) and some pair is allowed. Prefix-LM
  // alone is one predicate that is not all-false. Everything else is settled exhaustively.
  if (!(a.flags & FA_MASK_DOC)) {
    if (!(a.flags & FA_MASK_PREFIX_LM)) return 1;
    if (!(a.flags & FA_MASK_WINDOW)) return 1;
  }
  return 3;
}

__global__ __launch_bounds__(256) void bm_classify(BlockMaskArgs a) {
  const int qb = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_qdoc[128];
  __shared__ int s_kvdoc[128];
  __shared__ int s_amb[256];
  __shared__ int s_res[256];
  __shared__ int s_namb;
  __shared__ int s_wf[4], s_wp[4];

  const int q0 = qb * a.BQ, q1 = min(a.Lq, q0 + a.BQ);
  const bool doc = (a.flags & FA_MASK_DOC) != 0;
  const MaskSpec ms{a.flags, a.window, a.prefix_len};
  int qmin = 0, qmax = 0;
  if (doc) {
    qmin = a.qsum[2 * (b * a.nqb + qb)];
    qmax = a.qsum[2 * (b * a.nqb + qb) + 1];
    if (tid < a.BQ) s_qdoc[tid] = (q0 + tid < q1) ? a.q_doc[(int64_t)b * a.Lq + q0 + tid] : 0;
  }
  const int64_t row = (int64_t)b * a.nqb + qb;  // Hm = 1
  int* full_idx = a.full_idx + row * a.nkvb;
  int* part_idx = a.kv_idx + row * a.nkvb;
  int nfull = 0, npart = 0;

  for (int c0 = 0; c0 < a.nkvb; c0 += 256) {
    const int kb = c0 + tid;
    int cls = -1;
    if (kb < a.nkvb) {
      const int k0 = kb * a.BK, k1 = min(a.Lkv, k0 + a.BK);
      int kmin = 0, kmax = 0;
      if (doc) {
        kmin = a.kvsum[2 * (b * a.nkvb + kb)];
        kmax = a.kvsum[2 * (b * a.nkvb + kb) + 1];
      }
      cls = classify_closed(a, q0, q1, k0, k1, qmin, qmax, kmin, kmax);
    }
    if (tid == 0) s_namb = 0;
    __syncthreads();
    if (cls == 3) s_amb[atomicAdd(&s_namb, 1)] = kb;
    __syncthreads();
    const int namb = s_namb;
    for (int ai = 0; ai < namb; ++ai) {
      const int kbA = s_amb[ai];
      const int k0 = kbA * a.BK, k1 = min(a.Lkv, k0 + a.BK);
      if (doc && tid < a.BK) s_kvdoc[tid] = (k0 + tid < k1) ? a.kv_doc[(int64_t)b * a.Lkv + k0 + tid] : 0;
      __syncthreads();
      bool any = false;
      for (int e = tid; e < a.BQ * a.BK; e += 256) {
        const int ii = e / a.BK, jj = e % a.BK;
        const int i = q0 + ii, j = k0 + jj;
        if (i < q1 && j < k1) any = any || mask_pair(ms, i, j, doc ? s_qdoc[ii] : 0, doc ? s_kvdoc[jj] : 0);
      }
      any = __syncthreads_or(any);
      if (tid == 0) s_res[kbA - c0] = any ? 1 : 0;
      __syncthreads();
    }
    if (cls == 3) cls = s_res[tid];

    // Ascending compaction: ballot within each wave, then across the 4 waves.
    const bool isF = cls == 2, isP = cls == 1;
    const uint64_t bf = __ballot(isF), bp = __ballot(isP);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int pf = __popcll(bf & below), pp = __popcll(bp & below);
    if (lane == 0) {
      s_wf[wave] = __popcll(bf);
      s_wp[wave] = __popcll(bp);
    }
    __syncthreads();
    int basef = nfull, basep = npart, totf = 0, totp = 0;
    for (int w = 0; w < 4; ++w) {
      if (w < wave) {
        basef += s_wf[w];
        basep += s_wp[w];
      }
      totf += s_wf[w];
      totp += s_wp[w];
    }
    if (isF) full_idx[basef + pf] = kb;
    if (isP) part_idx[basep + pp] = kb;
    nfull += totf;
    npart += totp;
    __syncthreads();
  }
  for (int j = nfull + tid; j < a.nkvb; j += 256) full_idx[j] = 0;
  for (int j = npart + tid; j < a.nkvb; j += 256) part_idx[j] = 0;
  if (tid == 0) {
    a.full_num[row] = nfull;
    a.kv_num[row] = npart;
  }
}

hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t stream) {
  if (a.nqb == 0) return hipSuccess;
  if (a.flags & FA_MASK_DOC) {
    const int n = a.B * (a.nqb + a.nkvb);
    hipLaunchKernelGGL(bm_summaries, dim3((n + 255) / 256), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bm_classify, dim3(a.nqb, a.Bm), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa

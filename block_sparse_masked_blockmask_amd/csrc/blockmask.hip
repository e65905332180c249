// BlockMask construction on the device (gfx950).
//
// FlexAttention guide, "Systems Mechanics", item 1: the mask predicate is evaluated over each
// tile's bounding box; all-true tiles are full, all-false tiles are empty (never visited), the
// rest are partial. Here the box is the tile's in-range pairs. Each (mask row, query block) row
// is classified by one workgroup, 2048 kv blocks per pass:
//   1. closed forms (tile_class.h) decide most tiles exactly from corner tests and per-block
//      document-id summaries [min, max, dense]; one kv block per thread and round, so the
//      16-byte summaries are read with fully coalesced loads;
//   2. tiles that the closed forms cannot settle are evaluated pair by pair by the whole
//      workgroup (exact for any ids, sorted or not);
//   3. ordered compaction: wave w owns kv blocks [512 w, 512 w + 512) of the pass; ballots of
//      the classes (kept in LDS) give each lane its rank, wave totals give each wave its base,
//      so the full and partial lists are written in ascending order with coalesced stores.
// The unused tails of both lists are zeroed.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"
#include "tile_class.h"

namespace fa {

namespace {

constexpr int kChunk = 2048;  // kv blocks classified per pass of a workgroup
constexpr int kRounds = kChunk / 256;      // rounds of one kv block per thread
constexpr int kWaveRounds = kChunk / 4 / 64;  // rounds of one kv block per lane over a wave's quarter

__device__ __forceinline__ int wave_reduce_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ int wave_reduce_max(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}

}  // namespace

// One wave per (batch, block) of either side: [min id, max id, dense flag, 0].
__global__ __launch_bounds__(256) void bm_summaries(BlockMaskArgs a) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nq = a.B * a.nqb, nk = a.B * a.nkvb;
  if (w >= nq + nk) return;
  const int* ids;
  int lo, hi;
  int* dst;
  if (w < nq) {
    const int b = w / a.nqb, blk = w % a.nqb;
    ids = a.q_doc + (int64_t)b * a.Lq;
    lo = blk * a.BQ;
    hi = min(a.Lq, lo + a.BQ);
    dst = a.qsum + 4 * w;
  } else {
    const int u = w - nq;
    const int b = u / a.nkvb, blk = u % a.nkvb;
    ids = a.kv_doc + (int64_t)b * a.Lkv;
    lo = blk * a.BK;
    hi = min(a.Lkv, lo + a.BK);
    dst = a.kvsum + 4 * u;
  }
  int mn = INT_MAX, mx = INT_MIN;
  bool step_ok = true;
  for (int i = lo + lane; i < hi; i += 64) {
    const int d = ids[i];
    mn = min(mn, d);
    mx = max(mx, d);
    if (i > lo) {
      const int inc = d - ids[i - 1];
      step_ok = step_ok && (inc == 0 || inc == 1);
    }
  }
  mn = wave_reduce_min(mn);
  mx = wave_reduce_max(mx);
  const bool dense = __ballot(!step_ok) == 0;
  if (lane == 0) *(int4*)dst = make_int4(mn, mx, dense ? 1 : 0, 0);
}

__global__ __launch_bounds__(256) void bm_classify(BlockMaskArgs a) {
  const int qb = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_qdoc[256];
  __shared__ int s_kvdoc[128];
  __shared__ int s_amb[kChunk];
  __shared__ unsigned char s_cls[kChunk];
  __shared__ int s_namb;
  __shared__ int s_wtot[4];

  const int q0 = qb * a.BQ, q1 = min(a.Lq, q0 + a.BQ);
  const bool doc = (a.flags & FA_MASK_DOC) != 0;
  const MaskSpec ms{a.flags, a.window, a.prefix_len};
  int4 qs = make_int4(0, 0, 0, 0);
  if (doc) {
    qs = *(const int4*)(a.qsum + 4 * (b * a.nqb + qb));
    if (tid < a.BQ) s_qdoc[tid] = (q0 + tid < q1) ? a.q_doc[(int64_t)b * a.Lq + q0 + tid] : 0;
  }
  const int64_t row = (int64_t)b * a.nqb + qb;  // Hm = 1
  int* full_idx = a.full_idx + row * a.nkvb;
  int* part_idx = a.kv_idx + row * a.nkvb;
  int nfull = 0, npart = 0;  // wave-uniform running totals

  for (int c0 = 0; c0 < a.nkvb; c0 += kChunk) {
    // 1. closed forms, one kv block per thread and round.
    if (tid == 0) s_namb = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int loc = r * 256 + tid, kb = c0 + loc;
      int cls = 0;
      if (kb < a.nkvb) {
        const int k0 = kb * a.BK, k1 = min(a.Lkv, k0 + a.BK);
        int4 ks = make_int4(0, 0, 0, 0);
        if (doc) ks = *(const int4*)(a.kvsum + 4 * (b * a.nkvb + kb));
        cls = classify_closed(a.flags, a.window, a.prefix_len, q0, q1, k0, k1, qs.x, qs.y, qs.z, ks.x, ks.y, ks.z,
                              a.self_ids != 0);
        if (cls == 3) s_amb[atomicAdd(&s_namb, 1)] = loc;
      }
      s_cls[loc] = (unsigned char)cls;
    }
    __syncthreads();

    // 2. undecided tiles: every in-range pair, evaluated by the whole workgroup.
    const int namb = s_namb;
    for (int ai = 0; ai < namb; ++ai) {
      const int loc = s_amb[ai];
      const int k0 = (c0 + loc) * a.BK, k1 = min(a.Lkv, k0 + a.BK);
      if (doc && tid < a.BK) s_kvdoc[tid] = (k0 + tid < k1) ? a.kv_doc[(int64_t)b * a.Lkv + k0 + tid] : 0;
      __syncthreads();
      bool any = false;
      for (int e = tid; e < a.BQ * a.BK; e += 256) {
        const int ii = e / a.BK, jj = e % a.BK;
        const int i = q0 + ii, j = k0 + jj;
        if (i < q1 && j < k1) any = any || mask_pair(ms, i, j, doc ? s_qdoc[ii] : 0, doc ? s_kvdoc[jj] : 0);
      }
      any = __syncthreads_or(any);
      if (tid == 0) s_cls[loc] = any ? 1 : 0;
      __syncthreads();
    }

    // 3. ordered compaction (full and partial counts of a wave packed in one int).
    const int wb = wave * (kChunk / 4);
    int wcount = 0;
#pragma unroll
    for (int r = 0; r < kWaveRounds; ++r) {
      const int c = s_cls[wb + r * 64 + lane];
      wcount += __popcll(__ballot(c == 2)) + (__popcll(__ballot(c == 1)) << 16);
    }
    if (lane == 0) s_wtot[wave] = wcount;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t = s_wtot[w];
      if (w < wave) base += t;
      tot += t;
    }
    int pf = nfull + (base & 0xffff), pp = npart + (base >> 16);
#pragma unroll
    for (int r = 0; r < kWaveRounds; ++r) {
      const int loc = wb + r * 64 + lane;
      const int c = s_cls[loc];
      const uint64_t bf = __ballot(c == 2), bp = __ballot(c == 1);
      const uint64_t below = (1ull << lane) - 1;
      if (c == 2) full_idx[pf + __popcll(bf & below)] = c0 + loc;
      if (c == 1) part_idx[pp + __popcll(bp & below)] = c0 + loc;
      pf += __popcll(bf);
      pp += __popcll(bp);
    }
    nfull += tot & 0xffff;
    npart += tot >> 16;
    __syncthreads();  // s_namb, s_amb, s_cls and s_wtot are reused by the next pass
  }
  for (int j = nfull + tid; j < a.nkvb; j += 256) full_idx[j] = 0;
  for (int j = npart + tid; j < a.nkvb; j += 256) part_idx[j] = 0;
  if (tid == 0) {
    a.full_num[row] = nfull;
    a.kv_num[row] = npart;
  }
}

// Schedule of each mask row set (optional): its query blocks sorted by row_order_key, i.e. by
// decreasing cost. One workgroup of 1024 threads per row set sorts the keys in LDS with a
// bitonic network; in every stage each thread takes whole compare-exchange pairs (pair t joins
// index i, t with a zero inserted at bit log2(j), and i + j), so no thread idles.
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void bm_order(BlockMaskArgs a) {
  __shared__ unsigned s_key[kRowOrderMax];
  const int64_t row0 = (int64_t)blockIdx.x * a.nqb;
  int* order = a.row_order + row0;
  const int tid = threadIdx.x;
  if (a.nqb > kRowOrderMax) {
    for (int i = tid; i < a.nqb; i += kOrderThreads) order[i] = i;
    return;
  }
  int n = 2;
  while (n < a.nqb) n <<= 1;
  for (int i = tid; i < n; i += kOrderThreads)
    s_key[i] = i < a.nqb ? row_order_key(a.full_num[row0 + i], a.kv_num[row0 + i], i) : 0xffffffffu;
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = tid; t < n / 2; t += kOrderThreads) {
        const int i = 2 * t - (t & (j - 1)), l = i + j;
        const unsigned x = s_key[i], y = s_key[l];
        if ((x > y) == ((i & k) == 0)) {
          s_key[i] = y;
          s_key[l] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < a.nqb; i += kOrderThreads) order[i] = (int)(s_key[i] & kRowOrderQbMask);
}

hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t stream) {
  if (a.nqb == 0) return hipSuccess;
  if (a.flags & FA_MASK_DOC) {
    const int n = a.B * (a.nqb + a.nkvb);  // one wave each, four waves per workgroup
    hipLaunchKernelGGL(bm_summaries, dim3((n + 3) / 4), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bm_classify, dim3(a.nqb, a.Bm), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.row_order == nullptr) return e;
  hipLaunchKernelGGL(bm_order, dim3(a.Bm), dim3(kOrderThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_block_mask_order(const BlockMaskArgs& a, int nsets, hipStream_t stream) {
  if (nsets <= 0 || a.nqb <= 0) return hipSuccess;
  hipLaunchKernelGGL(bm_order, dim3(nsets), dim3(kOrderThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa

// BlockMask construction on the device (gfx950).
//
// FlexAttention guide, "Systems Mechanics", item 1: the mask predicate is evaluated over each
// tile's bounding box; all-true tiles are full, all-false tiles are empty (never visited), the
// rest are partial. Here the box is the tile's in-range pairs. Each (mask row, query block) row
// is classified by one workgroup:
//   1. closed forms decide most tiles exactly: the index predicates (causal, window, prefix-LM)
//      are monotone in q - kv or kv, so their all-true / all-false conditions are corner tests;
//      document ids use per-block summaries: [min, max] (equal single ids: full; disjoint:
//      empty) and a "dense" flag (consecutive ids differ by 0 or 1, so every id in [min, max]
//      occurs in the block; two dense blocks with overlapping ranges then share an id);
//   2. tiles that the closed forms cannot settle are evaluated pair by pair by the whole
//      workgroup (exact for any ids, sorted or not);
//   3. each thread owns a run of consecutive kv blocks; one block-wide scan of the per-thread
//      counts writes the full and partial lists in ascending order; their tails are zeroed.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"
#include "tile_class.h"

namespace fa {

namespace {

constexpr int kPerThread = 8;                 // kv blocks owned by one thread per chunk
constexpr int kChunk = 256 * kPerThread;      // kv blocks classified per pass of a workgroup

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

// One wave per (batch, block) of either side: [min id, max id, dense flag].
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
    dst = a.qsum + 3 * w;
  } else {
    const int u = w - nq;
    const int b = u / a.nkvb, blk = u % a.nkvb;
    ids = a.kv_doc + (int64_t)b * a.Lkv;
    lo = blk * a.BK;
    hi = min(a.Lkv, lo + a.BK);
    dst = a.kvsum + 3 * u;
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
  if (lane == 0) {
    dst[0] = mn;
    dst[1] = mx;
    dst[2] = dense ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void bm_classify(BlockMaskArgs a) {
  const int qb = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_qdoc[256];
  __shared__ int s_kvdoc[128];
  __shared__ int s_amb[kChunk];
  __shared__ unsigned char s_res[kChunk];
  __shared__ int s_namb;
  __shared__ int s_wtot[4];

  const int q0 = qb * a.BQ, q1 = min(a.Lq, q0 + a.BQ);
  const bool doc = (a.flags & FA_MASK_DOC) != 0;
  const MaskSpec ms{a.flags, a.window, a.prefix_len};
  int qmin = 0, qmax = 0, qdense = 0;
  if (doc) {
    const int* qs = a.qsum + 3 * (b * a.nqb + qb);
    qmin = qs[0];
    qmax = qs[1];
    qdense = qs[2];
    if (tid < a.BQ) s_qdoc[tid] = (q0 + tid < q1) ? a.q_doc[(int64_t)b * a.Lq + q0 + tid] : 0;
  }
  const int64_t row = (int64_t)b * a.nqb + qb;  // Hm = 1
  int* full_idx = a.full_idx + row * a.nkvb;
  int* part_idx = a.kv_idx + row * a.nkvb;
  int nfull = 0, npart = 0;

  for (int c0 = 0; c0 < a.nkvb; c0 += kChunk) {
    // 1. closed forms for this thread's run of kv blocks (summaries loaded up front).
    const int kb0 = c0 + tid * kPerThread;
    int kmn[kPerThread], kmx[kPerThread], kdn[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      kmn[j] = kmx[j] = kdn[j] = 0;
      if (doc && kb0 + j < a.nkvb) {
        const int* ks = a.kvsum + 3 * (b * a.nkvb + kb0 + j);
        kmn[j] = ks[0];
        kmx[j] = ks[1];
        kdn[j] = ks[2];
      }
    }
    if (tid == 0) s_namb = 0;
    __syncthreads();
    int cls[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int kb = kb0 + j;
      cls[j] = -1;
      if (kb < a.nkvb) {
        const int k0 = kb * a.BK, k1 = min(a.Lkv, k0 + a.BK);
        cls[j] = classify_closed(a.flags, a.window, a.prefix_len, q0, q1, k0, k1, qmin, qmax, qdense, kmn[j],
                                 kmx[j], kdn[j]);
        if (cls[j] == 3) s_amb[atomicAdd(&s_namb, 1)] = tid * kPerThread + j;
      }
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
      if (tid == 0) s_res[loc] = any ? 1 : 0;
      __syncthreads();
    }

    // 3. ascending compaction: exclusive scan of (full, partial) counts packed in one int.
    int packed = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if (cls[j] == 3) cls[j] = s_res[tid * kPerThread + j];
      packed += (cls[j] == 2 ? 1 : 0) + (cls[j] == 1 ? 0x10000 : 0);
    }
    int incl = packed;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o, 64);
      if (lane >= o) incl += up;
    }
    if (lane == 63) s_wtot[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wave) base += s_wtot[w];
      tot += s_wtot[w];
    }
    const int excl = base + incl - packed;
    int pf = nfull + (excl & 0xffff), pp = npart + (excl >> 16);
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if (cls[j] == 2) full_idx[pf++] = kb0 + j;
      if (cls[j] == 1) part_idx[pp++] = kb0 + j;
    }
    nfull += tot & 0xffff;
    npart += tot >> 16;
    __syncthreads();  // s_namb, s_amb, s_res and s_wtot are reused by the next chunk
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
    const int n = a.B * (a.nqb + a.nkvb);  // one wave each, four waves per workgroup
    hipLaunchKernelGGL(bm_summaries, dim3((n + 3) / 4), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bm_classify, dim3(a.nqb, a.Bm), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa

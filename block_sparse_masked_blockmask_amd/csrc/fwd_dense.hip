// bf16 forward for every-tile-full attention (no BlockMask: mask_kind NONE), gfx950, head dim 128,
// software-pipelined so that the vector work of one step overlaps the products of the next.
//
// The method is the forward of the FlexAttention guide ("The Core Design Principles"; with no
// mask_mod every tile is full, "Systems Mechanics" item 1): scores q.k/sqrt(d), the score_mod on
// every score, an online softmax over steps of 64 keys with intermediates kept on chip ("Fused
// Triton JIT Kernel Compilation", item 3).
//
// Operand formats are those of the block-sparse kernel (fwd.hip): each wave owns 32 queries;
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with Q^T held in registers; P^T stays in registers as the
// B operand of O^T = V^T P^T; V^T is read from the row-major V tile with ds_read_b64_tr_b16.
//
// The block-sparse kernel runs a step as S(n), then softmax(S(n)), then O += V(n)^T P(n): the
// exponentials wait for the products and the products for the exponentials. Here iteration n
// issues the 16 products of S(n+1) beside P(n) = exp2(S(n) - m) (its exponentials, row sums and
// bf16 packing), then the 16 products of O += V(n)^T P(n). The row maximum of S(n) and the lazy
// rescale come first in the iteration; the scores alternate between two register tiles.
//
// A workgroup is 8 waves (256 queries), one per CU at two waves per SIMD: the 8 waves share each
// K and V tile, which halves the L2-to-LDS traffic of two 4-wave workgroups (measured 5% faster).
// LDS: K slots for K(n+1) and K(n+2), V slots for V(n) and V(n+1), 16 KB each: iteration n waits
// for K(n+1) and V(n), passes one barrier, and refills the slots last read in iteration n-1. Each
// slot is an array of its own, named at compile time, so that the compiler waits for a transfer
// only before reading the slot it fills.
#include <hip/hip_runtime.h>

#include <climits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kDStep = 64;                 // keys per step
constexpr int kDStepBytes = kDStep * 256;  // one K or V step tile in LDS
constexpr float kDSlack = 8.0f;            // lazy maximum: rescale only past this (log2 units)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

__shared__ __attribute__((aligned(1024))) unsigned char d_k0[kDStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char d_k1[kDStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char d_v0[kDStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char d_v1[kDStepBytes];

template <int B> __device__ __forceinline__ unsigned char* dkbuf() { return B == 0 ? d_k0 : d_k1; }
template <int B> __device__ __forceinline__ unsigned char* dvbuf() { return B == 0 ? d_v0 : d_v1; }

__device__ __forceinline__ void ddma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}

__device__ __forceinline__ void wait_all_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct DLane {
  int wave, lane, hl, lq;
  int qi;
  bool q_in;
  float slope;
  const __bf16* kp;
  const __bf16* vp;
  int koff, voff;  // element offset of this lane's 16-byte DMA chunk in its first row
  int kx0, vx0;    // byte offsets of this lane's first K-operand and transposed V reads in a tile
};

// Score transform of one product (log2 domain), as in the block-sparse kernel: without a
// score_mod the scale is folded into the exponent later; ALiBi then soft-cap otherwise, with the
// constants folded on the host (FwdArgs::sc_in, sc_out, sc_out2, slope_mul).
template <int SCORE>
__device__ __forceinline__ float dscore(const FwdArgs& a, float acc, int qi, int kv, float slope) {
  if constexpr (SCORE == 0) {
    return acc;
  } else if constexpr (SCORE == FA_SCORE_ALIBI) {
    return fmaf(-slope, fabsf((float)(qi - kv)), acc * a.scale_log2);
  } else {
    float u = acc * a.sc_in;
    if constexpr (SCORE & FA_SCORE_ALIBI) u = fmaf(-slope, fabsf((float)(qi - kv)), u);
    return fmaf(a.sc_out2, __builtin_amdgcn_rcpf(1.0f + fast_exp2(u)), a.sc_out);
  }
}

// Soft-cap only: r = 1 / (1 + 2^u), the logit being sc_out + sc_out2 * r with sc_out2 < 0 (as in
// the block-sparse kernel's softcap_r). The tile keeps r; the row maximum comes from the row
// minimum of r, and the exponent argument is r * sc_out2 + (sc_out - m). Masked: r = +inf.
template <int SCORE>
__device__ __forceinline__ float dscore_r(const FwdArgs& a, float acc, int qi, int kv, float slope) {
  float u = acc * a.sc_in;
  if constexpr (SCORE & FA_SCORE_ALIBI) u = fmaf(-slope, fabsf((float)(qi - kv)), u);
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(u));
}

// One step's K or V tile: 16 one-KB segments (4 rows each); wave w issues segments 8 i + w.
// Rows past the last key are clamped to it (finite data, masked).
template <bool K_SIDE>
__device__ __forceinline__ void issue_tile(const FwdArgs& a, const DLane& c, int kv0, unsigned char* dst) {
  // The tile's first row is a uniform address; each lane adds a 32-bit byte offset.
  const int64_t sl = K_SIDE ? a.k_sl : a.v_sl;
  const char* base = (const char*)(K_SIDE ? c.kp : c.vp) + (int64_t)kv0 * sl * 2;
  if (kv0 + kDStep <= a.Lkv) {
    const unsigned off = (unsigned)(K_SIDE ? c.koff : c.voff) * 2u;
#pragma unroll
    for (int i = 0; i < 2; ++i) ddma16(base + (int64_t)(32 * i) * sl * 2 + off, dst + (8 * i + c.wave) * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = 8 * i + c.wave;
      const int r = seg * 4 + (c.lane >> 4);
      const int ch = (c.lane & 15) ^ swz(r);
      const int kr = min(kv0 + r, a.Lkv - 1) - kv0;
      ddma16(base + (unsigned)(kr * (int)sl * 2 + ch * 16), dst + seg * 1024);
    }
  }
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS operand reads are issued this many products before the product that uses them.
constexpr int kReadAhead = 4;

struct DState {
  f32x16 o[4];
  float m, l[4];
};

// S^T = K Q^T for one step (two 32-key sub-blocks), K from LDS tile sK.
__device__ __forceinline__ void dscores(const unsigned char* sK, int kx0, const bf16x8 (&q)[8], f32x16 (&s)[2]) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bf16x8 kf = *(const bf16x8*)(sK + nb * 32 * 256 + (kx0 ^ (32 * ks)));
      s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q[ks], ks ? s[nb] : f32x16{}, 0, 0, 0);
    }
  }
}

// Row maximum of step kv0's scores in s (score transform and, TAIL, the key bound of the ragged
// last step applied in place), the lazy rescale, then S(n+1) into sn from K tile sK (HAS_NEXT)
// issued beside P = exp2(S scale - m) into pb with its row sums.
template <int SCORE, bool HAS_NEXT, bool TAIL>
__device__ __forceinline__ void dense_part_a(const FwdArgs& a, const DLane& c, const bf16x8 (&qreg)[8], DState& st,
                                             f32x16 (&s)[2], f32x16 (&sn)[2], bf16x8 (&pb)[2][2], int kv0,
                                             const unsigned char* sK) {
  int kx0 = c.kx0;
  asm volatile("" : "+v"(kx0));
  constexpr bool CAP = (SCORE & FA_SCORE_SOFTCAP) != 0;
  float mx = CAP ? INFINITY : -INFINITY;  // CAP: row minimum of r
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kv0 + nb * 32 + (i >> 2) * 8 + c.hl * 4 + (i & 3);
      float x = CAP ? dscore_r<SCORE>(a, s[nb][i], c.qi, key, c.slope) : dscore<SCORE>(a, s[nb][i], c.qi, key, c.slope);
      if constexpr (TAIL) x = key < a.Lkv ? x : (CAP ? INFINITY : -INFINITY);
      s[nb][i] = x;
      mx = CAP ? fminf(mx, x) : fmaxf(mx, x);
    }
  }
  mx = CAP ? fmaf(a.sc_out2, half_swap_min(mx), a.sc_out) : half_swap_max(mx);
  const float scale = SCORE == 0 ? a.scale_log2 : 1.0f;
  const float m_cand = fmaxf(st.m, mx * scale);
  const bool raise = m_cand > st.m + kDSlack;
  if (__builtin_amdgcn_readfirstlane(__ballot(raise) != 0)) {
    const float m_new = raise ? m_cand : st.m;
    const float alpha = raise ? fast_exp2(st.m - m_new) : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) st.l[j] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[db] *= alpha;
    st.m = m_new;
  }
  const float neg_m = -st.m;
  const float cap_off = a.sc_out - st.m;
  if constexpr (HAS_NEXT) {
    // 16 products of S(n+1) in a fixed order (channel block k / 2, sub-block k % 2), each K
    // fragment read kReadAhead products ahead, and beside product k the exponentials of elements
    // 2k and 2k+1 of P(n) and the sums and bf16 packing of elements 2k-2 and 2k-1.
    bf16x8 kf[16];
    float pe[32];
    static_for<16>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k == 0) {
        static_for<kReadAhead + 1>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          kf[r] = *(const bf16x8*)(sK + (r & 1) * 32 * 256 + (kx0 ^ (32 * (r >> 1))));
        });
      } else if constexpr (k + kReadAhead < 16) {
        constexpr int r = k + kReadAhead;
        kf[r] = *(const bf16x8*)(sK + (r & 1) * 32 * 256 + (kx0 ^ (32 * (r >> 1))));
      }
      sn[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qreg[k >> 1], k >= 2 ? sn[k & 1] : f32x16{}, 0, 0,
                                                          0);
      static_for<2>([&](auto ec) {
        constexpr int e = 2 * k + decltype(ec)::value;
        pe[e] = fast_exp2(CAP ? fmaf(s[e >> 4][e & 15], a.sc_out2, cap_off) : fmaf(s[e >> 4][e & 15], scale, neg_m));
      });
      if constexpr (k > 0) {
        static_for<2>([&](auto ec) {
          constexpr int e = 2 * k - 2 + decltype(ec)::value;
          st.l[e & 3] += pe[e];
          pb[e >> 4][(e >> 3) & 1][e & 7] = (__bf16)pe[e];
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<2>([&](auto ec) {
      constexpr int e = 30 + decltype(ec)::value;
      st.l[e & 3] += pe[e];
      pb[e >> 4][(e >> 3) & 1][e & 7] = (__bf16)pe[e];
    });
  } else {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(CAP ? fmaf(s[nb][i], a.sc_out2, cap_off) : fmaf(s[nb][i], scale, neg_m));
        st.l[i & 3] += p;
        pb[nb][i >> 3][i & 7] = (__bf16)p;
      }
    }
  }
}

// O^T += V^T P^T from V tile sV: 16 products in a fixed order (channel block k / 4, sub-block
// (k / 2) % 2, 16-key group k % 2), each V fragment read kReadAhead products ahead.
__device__ __forceinline__ void dense_part_b(const DLane& c, DState& st, const bf16x8 (&pb)[2][2],
                                             const unsigned char* sV) {
  int vx0 = c.vx0;
  asm volatile("" : "+v"(vx0));
  bf16x8 vf[16];
  auto read = [&](auto rc) {
    constexpr int r = decltype(rc)::value;
    constexpr int db = r >> 2, nb = (r >> 1) & 1, h = r & 1;
    constexpr int rows = (nb * 32 + h * 16) * 256;
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(sV + rows + (vx0 ^ (64 * db))));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(sV + rows + (vx0 ^ (64 * db + 2080))));
    vf[r] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  __builtin_amdgcn_sched_barrier(0);
  static_for<16>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) {
      static_for<kReadAhead + 1>(read);
    } else if constexpr (k + kReadAhead < 16) {
      read(std::integral_constant<int, k + kReadAhead>{});
    }
    constexpr int db = k >> 2, nb = (k >> 1) & 1, h = k & 1;
    st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[k], pb[nb][h], st.o[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Iteration n: KB = (n + 1) & 1 is the slot of K(n+1) (S(n+1) is read from it, K(n+2) refills the
// other K slot) and of V(n+1) (V(n) is read from the other V slot). s holds S(n), sn receives
// S(n+1). HAS_NEXT: step n+1 exists; TAIL: step n is the ragged last step.
template <int SCORE, int KB, bool HAS_NEXT, bool TAIL>
__device__ __forceinline__ void dense_step(const FwdArgs& a, const DLane& c, const bf16x8 (&qreg)[8], DState& st,
                                           f32x16 (&s)[2], f32x16 (&sn)[2], int n, int nsteps) {
  wait_all_vmem();
  __syncthreads();
  if (n + 2 < nsteps) issue_tile<true>(a, c, (n + 2) * kDStep, dkbuf<KB ^ 1>());
  if (n + 1 < nsteps) issue_tile<false>(a, c, (n + 1) * kDStep, dvbuf<KB>());
  bf16x8 pb[2][2];
  dense_part_a<SCORE, HAS_NEXT, TAIL>(a, c, qreg, st, s, sn, pb, n * kDStep, dkbuf<KB>());
  __builtin_amdgcn_sched_barrier(0);
  dense_part_b(c, st, pb, dvbuf<KB ^ 1>());
}

}  // namespace

template <int SCORE>
__global__ __launch_bounds__(512, 1) void fwd_bf16_dense_kernel(FwdArgs a) {
  // Work order (as the block-sparse kernel without a schedule): each XCD takes a contiguous
  // range of work items; query heads of one kv head fastest, then query blocks from the last,
  // then the (batch, kv head) pairs, permuted so that every XCD mixes batches.
  int w = xcd_remap(blockIdx.x, a.total_wg);
  const int g = w % a.group;
  w /= a.group;
  const int qb = a.nqb - 1 - w % a.nqb;
  w /= a.nqb;
  const int npair = a.B * a.Hkv;
  const int q8 = npair / 8, r8 = npair % 8;
  int xc, xk;
  if (w < r8 * (q8 + 1)) {
    xc = w / (q8 + 1);
    xk = w % (q8 + 1);
  } else {
    xc = r8 + (w - r8 * (q8 + 1)) / q8;
    xk = (w - r8 * (q8 + 1)) % q8;
  }
  const int pair = 8 * xk + xc;
  const int hkv = pair % a.Hkv, b = pair / a.Hkv;
  const int hq = hkv * a.group + g;

  DLane c;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.lane = threadIdx.x & 63;
  c.hl = c.lane >> 5;
  c.lq = c.lane & 31;
  c.qi = qb * 256 + c.wave * 32 + c.lq;
  c.q_in = c.qi < a.Lq;
  c.kp = (const __bf16*)a.k + b * a.k_sb + hkv * a.k_sh;
  c.vp = (const __bf16*)a.v + b * a.v_sb + hkv * a.v_sh;
  c.kx0 = tile_off(c.lq, c.hl);
  {
    const int g16 = c.lane >> 4, s16 = c.lane & 15;
    const int d = 16 * (g16 & 1) + 4 * (s16 & 3);
    const int r0 = (g16 >> 1) * 4 + (s16 >> 2);
    c.vx0 = tile_off(r0, d >> 3) + (d & 7) * 2;
  }
  {
    const int r = c.wave * 4 + (c.lane >> 4);
    const int ch = (c.lane & 15) ^ swz(r);
    c.koff = r * (int)a.k_sl + ch * 8;
    c.voff = r * (int)a.v_sl + ch * 8;
  }
  c.slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[hq] * a.slope_mul : 0.f;

  // Q^T as the B operand: this lane's query row, channels 16 ks + 8 hl .. + 8; zero past the last
  // query.
  const __bf16* qp = (const __bf16*)a.q + b * a.q_sb + hq * a.q_sh;
  const int qi_c = min(c.qi, a.Lq - 1);
  bf16x8 qreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qreg[ks] = *(const bf16x8*)(qp + (int64_t)qi_c * a.q_sl + ks * 16 + c.hl * 8);
  if (!c.q_in) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = bf16x8{};
  }

  DState st;
#pragma unroll
  for (int db = 0; db < 4; ++db) st.o[db] = f32x16{};
  st.m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) st.l[j] = 0.f;

  const int nsteps = (a.Lkv + kDStep - 1) / kDStep;
  const bool ragged = (a.Lkv % kDStep) != 0;
  f32x16 s[2], s2[2];  // score tiles of alternate steps
  if (nsteps > 0) {
    // Prologue: K(0), V(0), K(1); S(0) once K(0) is in.
    issue_tile<true>(a, c, 0, d_k0);
    issue_tile<false>(a, c, 0, d_v0);
    if (nsteps > 1) issue_tile<true>(a, c, kDStep, d_k1);
    wait_all_vmem();
    __syncthreads();
    int kx0 = c.kx0;
    asm volatile("" : "+v"(kx0));
    dscores(d_k0, kx0, qreg, s);
  }
  // Step n reads K(n+1) from K slot (n + 1) & 1 and V(n) from V slot n & 1. In the loop neither
  // step n nor step n+1 is the last.
  int n = 0;
  for (; n + 2 < nsteps; n += 2) {
    dense_step<SCORE, 1, true, false>(a, c, qreg, st, s, s2, n, nsteps);
    dense_step<SCORE, 0, true, false>(a, c, qreg, st, s2, s, n + 1, nsteps);
  }
  // One or two steps remain (n even, S(n) in s); the last may be ragged.
  if (n + 1 < nsteps) {
    dense_step<SCORE, 1, true, false>(a, c, qreg, st, s, s2, n, nsteps);
    if (ragged) dense_step<SCORE, 0, false, true>(a, c, qreg, st, s2, s, n + 1, nsteps);
    else dense_step<SCORE, 0, false, false>(a, c, qreg, st, s2, s, n + 1, nsteps);
  } else if (n < nsteps) {
    if (ragged) dense_step<SCORE, 1, false, true>(a, c, qreg, st, s, s2, n, nsteps);
    else dense_step<SCORE, 1, false, false>(a, c, qreg, st, s, s2, n, nsteps);
  }
  wait_all_vmem();  // no transfer may outlive the workgroup's LDS

  // Epilogue: O / l in bf16 and the natural-log lse (l = 0 only without keys: O = 0, -inf).
  const float l_tot = half_swap_sum((st.l[0] + st.l[1]) + (st.l[2] + st.l[3]));
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (c.q_in) {
    __bf16* op = (__bf16*)a.o + b * a.o_sb + hq * a.o_sh + (int64_t)c.qi * a.o_sl;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 o4;
        o4[0] = (__bf16)(st.o[db][gq * 4 + 0] * inv);
        o4[1] = (__bf16)(st.o[db][gq * 4 + 1] * inv);
        o4[2] = (__bf16)(st.o[db][gq * 4 + 2] * inv);
        o4[3] = (__bf16)(st.o[db][gq * 4 + 3] * inv);
        *(bf16x4*)(op + db * 32 + gq * 8 + c.hl * 4) = o4;
      }
    }
    if (a.lse && c.hl == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Lq + c.qi] = l_tot > 0.f ? (st.m + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_fwd_dense(const FwdArgs& a, int score, hipStream_t stream) {
  if (a.total_wg == 0) return hipSuccess;
  const dim3 grid(a.total_wg), block(512);
  switch (score) {
    case 0: hipLaunchKernelGGL((fwd_bf16_dense_kernel<0>), grid, block, 0, stream, a); break;
    case FA_SCORE_ALIBI: hipLaunchKernelGGL((fwd_bf16_dense_kernel<FA_SCORE_ALIBI>), grid, block, 0, stream, a); break;
    case FA_SCORE_SOFTCAP: hipLaunchKernelGGL((fwd_bf16_dense_kernel<FA_SCORE_SOFTCAP>), grid, block, 0, stream, a); break;
    default:
      hipLaunchKernelGGL((fwd_bf16_dense_kernel<FA_SCORE_ALIBI | FA_SCORE_SOFTCAP>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace fa

// bf16 block-sparse forward with a software-pipelined step, gfx950, head dim 128, for masks whose
// allowed keys of a query form one interval (causal, sliding window, prefix-LM, or none).
//
// Method (FlexAttention guide): the forward of fwd.hip. Full tiles are computed without mask
// evaluation, partial tiles with it, and empty tiles are never visited ("Systems Mechanics",
// item 1); an online softmax over the visited tiles keeps the scores on chip ("Fused Triton JIT
// Kernel Compilation", item 3).
//
// The step is that of the every-tile-full kernel (fwd_dense.hip): iteration n takes the row
// maximum of S(n) and the lazy rescale, issues the 16 products of S(n+1) beside the exponentials,
// row sums and bf16 packing of P(n), then the 16 products of O += V(n)^T P(n). Here the steps come
// from the BlockMask's tile lists (full tiles first, then partial ones), and on a partial tile or
// the ragged last step the key interval of each query masks S(n) before its maximum is taken. The
// score_mod's vector work for S(n+1) runs beside the P(n).V(n) products, so iteration n starts
// from transformed scores.
// Unlike fwd.hip, a wave does not skip the 32x32 sub-blocks that its mask leaves empty: their
// products run and their probabilities come out exactly 0.
//
// A workgroup is 4 waves (the BlockMask's 128-query block; each wave owns 32 queries), two
// workgroups per CU. LDS: K slots for K(n+1) and K(n+2), V slots for V(n) and V(n+1), 16 KB each,
// every slot a distinct array named at compile time (the compiler then waits for a transfer only
// before reading the slot it fills). Iteration n waits for K(n+1) and V(n), passes one barrier and
// refills the slots last read in iteration n-1.
#include <hip/hip_runtime.h>

#include <climits>
#include <utility>

#include "device_common.h"
#include "launch.h"
#include "work_order.h"

namespace fa {

namespace {

constexpr int kPStep = 64;                 // keys per step
constexpr int kPStepBytes = kPStep * 256;  // one K or V step tile in LDS
constexpr float kPSlack = 8.0f;            // lazy maximum: rescale only past this (log2 units)
constexpr int kPReadAhead = 4;             // LDS operand reads issued this many products ahead

typedef __attribute__((address_space(3))) void lds_void_p;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_p;

__shared__ __attribute__((aligned(1024))) unsigned char p_k0[kPStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char p_k1[kPStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char p_v0[kPStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char p_v1[kPStepBytes];

template <int B> __device__ __forceinline__ unsigned char* pkbuf() { return B == 0 ? p_k0 : p_k1; }
template <int B> __device__ __forceinline__ unsigned char* pvbuf() { return B == 0 ? p_v0 : p_v1; }

__device__ __forceinline__ void pdma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_p*)lds, 16, 0, 0);
}

__device__ __forceinline__ void pwait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct PLane {
  int wave, lane, hl;
  int qi;
  bool q_in;
  float slope;
  const __bf16* kp;
  const __bf16* vp;
  int koff, voff;  // element offset of this lane's 16-byte transfer chunk in its first row
  int kx0, vx0;    // byte offsets of this lane's first K-operand and transposed V reads in a tile
};

// One step of the list: its first key and its kind (0: full tile; 1: partial tile or ragged last
// step, the mask is evaluated; 2: a list entry outside the key blocks, every score masked).
struct PStep {
  int kv0, kind;
};

// Score transform of one product in the log2 domain (as score_log2 in fwd.hip): without a
// score_mod the scale is folded into the exponent later; ALiBi then soft-cap otherwise.
template <int SCORE>
__device__ __forceinline__ float pscore(const FwdArgs& a, float acc, int qi, int kv, float slope) {
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

// Soft-cap: the tile keeps r = 1 / (1 + 2^u), the logit being sc_out + sc_out2 * r with
// sc_out2 < 0, so the row maximum comes from the row minimum of r and the exponent argument is
// r * sc_out2 + (sc_out - m). A masked score has r = +inf.
template <int SCORE>
__device__ __forceinline__ float pscore_r(const FwdArgs& a, float acc, int qi, int kv, float slope) {
  float u = acc * a.sc_in;
  if constexpr (SCORE & FA_SCORE_ALIBI) u = fmaf(-slope, fabsf((float)(qi - kv)), u);
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(u));
}

// One step's K or V tile: 16 one-KB segments (4 rows each); wave w issues segments 4 i + w, rows
// 16 i + 4 w + lane / 16. The swizzle depends on the row modulo 16 only, so the four segments of a
// wave share the lane's chunk offset. Rows past the last key are clamped to it (finite data, masked).
template <bool K_SIDE>
__device__ __forceinline__ void ptile(const FwdArgs& a, const PLane& c, int kv0, unsigned char* dst) {
  const int64_t sl = K_SIDE ? a.k_sl : a.v_sl;
  const char* base = (const char*)(K_SIDE ? c.kp : c.vp) + (int64_t)kv0 * sl * 2;
  if (kv0 + kPStep <= a.Lkv) {
    const unsigned off = (unsigned)(K_SIDE ? c.koff : c.voff) * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) pdma16(base + (int64_t)(16 * i) * sl * 2 + off, dst + (4 * i + c.wave) * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int seg = 4 * i + c.wave;
      const int r = seg * 4 + (c.lane >> 4);
      const int ch = (c.lane & 15) ^ swz(r);
      const int kr = min(kv0 + r, a.Lkv - 1) - kv0;
      pdma16(base + (int64_t)kr * sl * 2 + ch * 16, dst + seg * 1024);
    }
  }
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at compile time.
template <typename F, int... I>
__device__ __forceinline__ void pstatic_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void pstatic_for(F&& f) {
  pstatic_for_impl(f, std::make_integer_sequence<int, N>{});
}

struct PState {
  f32x16 o[4];
  float m, l[4];
};

// S^T = K Q^T for one step (two 32-key sub-blocks), K from LDS tile sK.
__device__ __forceinline__ void pscores(const unsigned char* sK, int kx0, const bf16x8 (&q)[8], f32x16 (&s)[2]) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bf16x8 kf = *(const bf16x8*)(sK + nb * 32 * 256 + (kx0 ^ (32 * ks)));
      s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q[ks], ks ? s[nb] : f32x16{}, 0, 0, 0);
    }
  }
}

// Score transform of one element of a step's S (as score_log2 in fwd.hip, log2 domain): the raw
// product without a score_mod (the scale is folded into the exponent), r with the soft-cap
// (pscore_r), the logit with ALiBi alone. Element i of sub-block nb holds key
// kv0 + nb*32 + (i/4)*8 + hl*4 + i%4.
template <int SCORE>
__device__ __forceinline__ float ptransform(const FwdArgs& a, const PLane& c, float acc, int kv0, int e) {
  const int key = kv0 + (e >> 4) * 32 + ((e & 15) >> 2) * 8 + c.hl * 4 + (e & 3);
  if constexpr (SCORE == 0) return acc;
  else if constexpr ((SCORE & FA_SCORE_SOFTCAP) != 0) return pscore_r<SCORE>(a, acc, c.qi, key, c.slope);
  else return pscore<SCORE>(a, acc, c.qi, key, c.slope);
}

// Step cur's transformed scores in s: the mask (partial tiles, the ragged last step, skipped
// entries), the row maximum and the lazy rescale, then S(n+1) into sn from K tile sK (HAS_NEXT)
// issued beside P = exp2(S - m) into pb with its row sums.
template <int SCORE, bool HAS_NEXT>
__device__ __forceinline__ void pipe_part_a(const FwdArgs& a, const PLane& c, const bf16x8 (&qreg)[8], PState& st,
                                            f32x16 (&s)[2], f32x16 (&sn)[2], bf16x8 (&pb)[2][2], const PStep& cur,
                                            const unsigned char* sK) {
  int kx0 = c.kx0;
  asm volatile("" : "+v"(kx0));
  constexpr bool CAP = (SCORE & FA_SCORE_SOFTCAP) != 0;
  if (cur.kind != 0) {
    // The allowed keys [lo, hi) of this lane's query relative to each sub-block's first key of
    // the lane as one bitmask (bit off: offset off allowed, offsets 0..27); each score takes its
    // bit with a signed shift (0 or all ones) and keeps its own bits or those of the masked value.
    int lo, hi;
    key_interval(a, c.qi, lo, hi);
    if (cur.kind == 2) hi = lo;  // a skipped list entry: no key allowed
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int kbase = cur.kv0 + nb * 32 + c.hl * 4;
      const int l0 = min(max(lo - kbase, 0), 31), h0 = min(max(hi - kbase, 0), 31);
      const unsigned abits = ((1u << h0) - 1u) & ~((1u << l0) - 1u);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = (i >> 2) * 8 + (i & 3);
        constexpr unsigned kMasked = CAP ? 0x7f800000u : 0xff800000u;  // +inf (r) or -inf
        const int keep = (int)(abits << (31 - off)) >> 31;
        s[nb][i] = __int_as_float((__float_as_int(s[nb][i]) & keep) | (int)(kMasked & ~(unsigned)keep));
      }
    }
  }
  float mx = CAP ? INFINITY : -INFINITY;  // CAP: row minimum of r
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = CAP ? fminf(mx, s[nb][i]) : fmaxf(mx, s[nb][i]);
  }
  mx = CAP ? fmaf(a.sc_out2, half_swap_min(mx), a.sc_out) : half_swap_max(mx);
  const float scale = SCORE == 0 ? a.scale_log2 : 1.0f;
  const float m_cand = fmaxf(st.m, mx * scale);
  const bool raise = m_cand > st.m + kPSlack;
  if (__builtin_amdgcn_readfirstlane(__ballot(raise) != 0)) {
    // Rows that keep m (including rows still at -inf) get alpha = 1 exactly; a row raised from
    // -inf gets exp2(-inf) = 0.
    const float m_new = raise ? m_cand : st.m;
    const float alpha = raise ? fast_exp2(st.m - m_new) : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) st.l[j] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[db] *= alpha;
    st.m = m_new;
  }
  // A row with no allowed key so far keeps m = -inf: its masked scores give exp2(-inf) = 0.
  const float m_eff = st.m == -INFINITY ? 0.f : st.m;
  const float neg_m = -m_eff;
  const float cap_off = a.sc_out - m_eff;
  if constexpr (HAS_NEXT) {
    // 16 products of S(n+1) in a fixed order (channel block k / 2, sub-block k % 2), each K
    // fragment read kPReadAhead products ahead, and beside product k the exponentials of
    // elements 2k and 2k+1 of P(n) and the sums and bf16 packing of elements 2k-2 and 2k-1.
    bf16x8 kf[16];
    float pe[32];
    pstatic_for<16>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k == 0) {
        pstatic_for<kPReadAhead + 1>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          kf[r] = *(const bf16x8*)(sK + (r & 1) * 32 * 256 + (kx0 ^ (32 * (r >> 1))));
        });
      } else if constexpr (k + kPReadAhead < 16) {
        constexpr int r = k + kPReadAhead;
        kf[r] = *(const bf16x8*)(sK + (r & 1) * 32 * 256 + (kx0 ^ (32 * (r >> 1))));
      }
      sn[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qreg[k >> 1], k >= 2 ? sn[k & 1] : f32x16{}, 0, 0,
                                                          0);
      pstatic_for<2>([&](auto ec) {
        constexpr int e = 2 * k + decltype(ec)::value;
        pe[e] = fast_exp2(CAP ? fmaf(s[e >> 4][e & 15], a.sc_out2, cap_off) : fmaf(s[e >> 4][e & 15], scale, neg_m));
      });
      if constexpr (k > 0) {
        pstatic_for<2>([&](auto ec) {
          constexpr int e = 2 * k - 2 + decltype(ec)::value;
          st.l[e & 3] += pe[e];
          pb[e >> 4][(e >> 3) & 1][e & 7] = (__bf16)pe[e];
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    pstatic_for<2>([&](auto ec) {
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
// (k / 2) % 2, 16-key group k % 2), each V fragment read kPReadAhead products ahead. XFORM: beside
// product k, the score transform of elements 2k and 2k+1 of S(n+1) in sn (first key kv0n), so that
// the score_mod's vector work overlaps these products.
template <int SCORE, bool XFORM>
__device__ __forceinline__ void pipe_part_b(const FwdArgs& a, const PLane& c, PState& st, const bf16x8 (&pb)[2][2],
                                            const unsigned char* sV, f32x16 (&sn)[2], int kv0n) {
  int vx0 = c.vx0;
  asm volatile("" : "+v"(vx0));
  bf16x8 vf[16];
  auto read = [&](auto rc) {
    constexpr int r = decltype(rc)::value;
    constexpr int db = r >> 2, nb = (r >> 1) & 1, h = r & 1;
    constexpr int rows = (nb * 32 + h * 16) * 256;
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(sV + rows + (vx0 ^ (64 * db))));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(sV + rows + (vx0 ^ (64 * db + 2080))));
    vf[r] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  __builtin_amdgcn_sched_barrier(0);
  pstatic_for<16>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) {
      pstatic_for<kPReadAhead + 1>(read);
    } else if constexpr (k + kPReadAhead < 16) {
      read(std::integral_constant<int, k + kPReadAhead>{});
    }
    constexpr int db = k >> 2, nb = (k >> 1) & 1, h = k & 1;
    st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[k], pb[nb][h], st.o[db], 0, 0, 0);
    if constexpr (XFORM && SCORE != 0) {
      pstatic_for<2>([&](auto ec) {
        constexpr int e = 2 * k + decltype(ec)::value;
        sn[e >> 4][e & 15] = ptransform<SCORE>(a, c, sn[e >> 4][e & 15], kv0n, e);
      });
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Iteration n: KB = (n + 1) & 1 is the slot of K(n+1) (S(n+1) is read from it, K(n+2) refills the
// other K slot) and of V(n+1) (V(n) is read from the other V slot). s holds S(n) transformed, sn
// receives S(n+1) transformed. nxt and nxt2 are steps n+1 and n+2 (transferred only if they exist).
template <int SCORE, int KB, bool HAS_NEXT>
__device__ __forceinline__ void pipe_step(const FwdArgs& a, const PLane& c, const bf16x8 (&qreg)[8], PState& st,
                                          f32x16 (&s)[2], f32x16 (&sn)[2], const PStep& cur, const PStep& nxt,
                                          const PStep& nxt2, int n, int nsteps) {
  pwait_all();
  __syncthreads();
  if (n + 2 < nsteps) ptile<true>(a, c, nxt2.kv0, pkbuf<KB ^ 1>());
  if (n + 1 < nsteps) ptile<false>(a, c, nxt.kv0, pvbuf<KB>());
  bf16x8 pb[2][2];
  pipe_part_a<SCORE, HAS_NEXT>(a, c, qreg, st, s, sn, pb, cur, pkbuf<KB>());
  __builtin_amdgcn_sched_barrier(0);
  pipe_part_b<SCORE, HAS_NEXT>(a, c, st, pb, pvbuf<KB ^ 1>(), sn, nxt.kv0);
}

}  // namespace

template <int SCORE, int HALVES>
__global__ __launch_bounds__(256, 2) void fwd_bf16_pipe_kernel(FwdArgs a) {
  constexpr int TB = HALVES * kPStep;  // keys per BlockMask tile
  const WorkItem it = decode_work<0>(a, blockIdx.x);
  PLane c;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.lane = threadIdx.x & 63;
  c.hl = c.lane >> 5;
  const int lq = c.lane & 31;
  c.qi = it.qb * 128 + c.wave * 32 + lq;
  c.q_in = c.qi < a.Lq;
  c.kp = (const __bf16*)a.k + it.b * a.k_sb + it.hkv * a.k_sh;
  c.vp = (const __bf16*)a.v + it.b * a.v_sb + it.hkv * a.v_sh;
  c.kx0 = tile_off(lq, c.hl);
  {
    // In each 16-lane group, source lane s points at key row base + s/4, channels d0 + 4*(s%4).
    const int g16 = c.lane >> 4, s16 = c.lane & 15;
    const int d = 16 * (g16 & 1) + 4 * (s16 & 3);
    const int r0 = (g16 >> 1) * 4 + (s16 >> 2);
    c.vx0 = tile_off(r0, d >> 3) + (d & 7) * 2;
  }
  {
    const int r = c.wave * 4 + (c.lane >> 4);  // row of this lane in its first segment
    const int ch = (c.lane & 15) ^ swz(r);
    c.koff = r * (int)a.k_sl + ch * 8;
    c.voff = r * (int)a.v_sl + ch * 8;
  }
  c.slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[it.hq] * a.slope_mul : 0.f;

  // First-round loads, all issued before any is waited for: this lane's Q row, the BlockMask
  // counts and the first 64 entries of both index lists (index rows always hold n_kvb entries).
  const __bf16* qp = (const __bf16*)a.q + it.b * a.q_sb + it.hq * a.q_sh;
  const int qi_c = min(c.qi, a.Lq - 1);
  bf16x8 qreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qreg[ks] = *(const bf16x8*)(qp + (int64_t)qi_c * a.q_sl + ks * 16 + c.hl * 8);
  const int* full_row;
  const int* part_row;
  int nfull, npart, chunk_init;
  {
    const int bm = a.Bm == 1 ? 0 : it.b;
    const int hm = a.Hm == 1 ? 0 : it.hq;
    const int64_t row = ((int64_t)bm * a.Hm + hm) * a.nqb + it.qb;
    // Without lists (no BlockMask, or no key block) the list reads go to this head's first Q row
    // (256 bytes, always present when a workgroup runs) and are ignored.
    const int* dummy = (const int*)qp;
    const bool no_lists = a.all_full || a.nkvb == 0;
    full_row = no_lists ? dummy : a.full_idx + row * a.nkvb;
    part_row = no_lists ? dummy : a.kv_idx + row * a.nkvb;
    const int fn = *(a.all_full ? dummy : a.full_num + row);
    const int pn = *(a.all_full ? dummy : a.kv_num + row);
    const int lc = max(min(c.lane, a.nkvb - 1), 0);
    const int fch = full_row[lc];
    const int pch = part_row[lc];
    // Counts come from caller memory: clamp them so that a corrupt BlockMask cannot send the
    // kernel outside the index arrays.
    nfull = a.all_full ? a.nkvb : min(max(fn, 0), a.nkvb);
    npart = a.all_full ? 0 : min(max(pn, 0), a.nkvb);
    // Merge: entries of the full list, then of the partial list, with one cross-lane move.
    const int pmv = __shfl(pch, (c.lane - nfull) & 63, 64);
    chunk_init = c.lane < nfull ? fch : pmv;
  }
  if (!c.q_in) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = bf16x8{};
  }
  const int ntiles = nfull + npart;
  const int nsteps = ntiles * HALVES;

  // List entries, 64 per register: lane j holds the entry of tile chunk_base + j.
  int chunk_base = 0;
  int chunk = chunk_init;
  auto info = [&](int s) {
    PStep si{0, 2};
    const int t = s / HALVES;
    if (t >= chunk_base + 64) {  // next 64 list entries (once per 64 tiles)
      chunk_base = t & ~63;
      const int tt = chunk_base + c.lane;
      chunk = (a.all_full || tt >= ntiles) ? tt : (tt < nfull ? full_row[tt] : part_row[tt - nfull]);
    }
    const int kb = a.all_full ? t : __builtin_amdgcn_readlane(chunk, t - chunk_base);
    const int kv0 = kb * TB + (s % HALVES) * kPStep;
    // A corrupt index, or a half past the last key, is a step with every score masked.
    const bool ok = kb >= 0 && kb < a.nkvb && kv0 < a.Lkv;
    si.kv0 = ok ? kv0 : 0;
    si.kind = !ok ? 2 : (t >= nfull || kv0 + kPStep > a.Lkv) ? 1 : 0;
    return si;
  };

  PState st;
#pragma unroll
  for (int db = 0; db < 4; ++db) st.o[db] = f32x16{};
  st.m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) st.l[j] = 0.f;

  f32x16 s[2], s2[2];  // score tiles of alternate steps
  PStep cur{0, 2}, nxt{0, 2};
  if (nsteps > 0) {
    // Prologue: K(0), V(0), K(1); S(0) once K(0) is in. Without any step nothing is transferred.
    cur = info(0);
    ptile<true>(a, c, cur.kv0, p_k0);
    ptile<false>(a, c, cur.kv0, p_v0);
    if (nsteps > 1) {
      nxt = info(1);
      ptile<true>(a, c, nxt.kv0, p_k1);
    }
    pwait_all();
    __syncthreads();
    int kx0 = c.kx0;
    asm volatile("" : "+v"(kx0));
    pscores(p_k0, kx0, qreg, s);
#pragma unroll
    for (int e = 0; e < 32; ++e) s[e >> 4][e & 15] = ptransform<SCORE>(a, c, s[e >> 4][e & 15], cur.kv0, e);
  }
  int n = 0;
  // One iteration. The kind of step n (wave-uniform) decides whether its scores are masked; only
  // that pass is conditional (with two copies of the whole step the compiler kept the
  // accumulators in two register sets and spilled).
  auto step = [&](auto kbc, auto hasc, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr int KB = decltype(kbc)::value;
    constexpr bool HAS = decltype(hasc)::value;
    const PStep nxt2 = (n + 2 < nsteps) ? info(n + 2) : PStep{0, 2};
    pipe_step<SCORE, KB, HAS>(a, c, qreg, st, sc, sn, cur, nxt, nxt2, n, nsteps);
    cur = nxt;
    nxt = nxt2;
    ++n;
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using HasNext = std::true_type;
  using Last = std::false_type;
  // Step n reads K(n+1) from K slot (n + 1) & 1 and V(n) from V slot n & 1. In the loop neither
  // step n nor step n+1 is the last.
  while (n + 2 < nsteps) {
    step(K1{}, HasNext{}, s, s2);
    step(K0{}, HasNext{}, s2, s);
  }
  // One or two steps remain (n even, S(n) in s).
  if (n + 1 < nsteps) {
    step(K1{}, HasNext{}, s, s2);
    step(K0{}, Last{}, s2, s);
  } else if (n < nsteps) {
    step(K1{}, Last{}, s, s2);
  }
  pwait_all();  // no transfer may outlive the workgroup's LDS

  // Epilogue: O / l in bf16 and the natural-log lse (l = 0 for a row with no allowed key: O = 0,
  // lse = -inf).
  const float l_tot = half_swap_sum((st.l[0] + st.l[1]) + (st.l[2] + st.l[3]));
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  // O goes out through LDS, so that each store writes whole rows (from the registers, each
  // instruction wrote 16 bytes into each of 32 rows): waves 0-1 stage their 32 x 256-byte rows in
  // the first K slot, waves 2-3 in the first V slot (free once every wave is past its last step),
  // swizzled; each wave reads back only its own rows.
  __syncthreads();
  unsigned char* const ob = (c.wave < 2 ? p_k0 : p_v0) + (c.wave & 1) * (32 * 256);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      bf16x4 o4;
      o4[0] = (__bf16)(st.o[db][gq * 4 + 0] * inv);
      o4[1] = (__bf16)(st.o[db][gq * 4 + 1] * inv);
      o4[2] = (__bf16)(st.o[db][gq * 4 + 2] * inv);
      o4[3] = (__bf16)(st.o[db][gq * 4 + 3] * inv);
      *(bf16x4*)(ob + tile_off(lq, db * 4 + gq) + c.hl * 8) = o4;
    }
  }
  // Row r of the wave (4 rows per instruction), 16-byte chunk lane % 16.
  __bf16* const op0 = (__bf16*)a.o + it.b * a.o_sb + it.hq * a.o_sh;
  const int qw0 = it.qb * 128 + c.wave * 32;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 4 * j + (c.lane >> 4), ch = c.lane & 15;
    const bf16x8 v8 = *(const bf16x8*)(ob + tile_off(r, ch));
    if (qw0 + r < a.Lq) *(bf16x8*)(op0 + (int64_t)(qw0 + r) * a.o_sl + ch * 8) = v8;
  }
  if (c.q_in && a.lse && c.hl == 0)
    a.lse[((int64_t)it.b * a.Hq + it.hq) * a.Lq + c.qi] = l_tot > 0.f ? (st.m + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int HALVES>
static hipError_t launch_pipe_bk(const FwdArgs& a, int score, hipStream_t stream) {
  const dim3 grid(a.total_wg), block(256);
  switch (score) {
    case 0: hipLaunchKernelGGL((fwd_bf16_pipe_kernel<0, HALVES>), grid, block, 0, stream, a); break;
    case FA_SCORE_ALIBI:
      hipLaunchKernelGGL((fwd_bf16_pipe_kernel<FA_SCORE_ALIBI, HALVES>), grid, block, 0, stream, a);
      break;
    case FA_SCORE_SOFTCAP:
      hipLaunchKernelGGL((fwd_bf16_pipe_kernel<FA_SCORE_SOFTCAP, HALVES>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((fwd_bf16_pipe_kernel<FA_SCORE_ALIBI | FA_SCORE_SOFTCAP, HALVES>), grid, block, 0, stream,
                         a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_fwd_pipe(const FwdArgs& a, int kv_block, int score, hipStream_t stream) {
  if (a.total_wg == 0) return hipSuccess;
  return kv_block == 64 ? launch_pipe_bk<1>(a, score, stream) : launch_pipe_bk<2>(a, score, stream);
}

}  // namespace fa

// Block-sparse masked attention forward for gfx950 (CDNA4), head dim 128.
//
// Method (FlexAttention guide): scores q.k/sqrt(d) ("The Core Design Principles"), a
// score_mod applied to every score of a visited tile, a mask_mod evaluated only on partial
// tiles, full tiles computed without mask branches and empty tiles never visited ("Systems
// Mechanics", item 1), intermediate scores kept on chip ("Fused Triton JIT Kernel Compilation",
// item 3) by an online softmax over the visited tiles.
//
// Work decomposition: one workgroup of 4 waves per (batch, query head, 128-query block); wave w
// owns 32 queries. Each wave computes the TRANSPOSED score tile S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers), so every lane holds
// scores of a single query (lane % 32) and the row max / row sum are in-lane reductions plus one
// v_permlane32_swap between the two wave halves. The softmax numerators P^T are already in the
// B-operand layout of the second product O^T = V^T P^T, so they are converted to bf16 in
// registers; V^T's A operand is read from the row-major V tile with ds_read_b64_tr_b16.
//
// Accumulator layout (32x32 MFMA, confirmed by a probe on gfx950): element i of lane l holds
// row 8*(i/4) + 4*(l/32) + i%4 and column l%32. For S^T the row is the key, for O^T the
// head-dim channel.
#include <hip/hip_runtime.h>

#include <climits>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "work_order.h"

namespace fa {

namespace {

constexpr int kD = 128;
constexpr int kBQ = 128;

struct TileList {
  const int* full;
  const int* part;
  int nfull, npart;
};

__device__ __forceinline__ TileList tile_list(const FwdArgs& a, const WorkItem& it) {
  TileList t;
  if (a.all_full) {
    t.full = nullptr;
    t.part = nullptr;
    t.nfull = a.nkvb;
    t.npart = 0;
    return t;
  }
  const int bm = a.Bm == 1 ? 0 : it.b;
  const int hm = a.Hm == 1 ? 0 : it.hq;
  const int64_t row = ((int64_t)bm * a.Hm + hm) * a.nqb + it.qb;
  t.full = a.full_idx + row * a.nkvb;
  t.part = a.kv_idx + row * a.nkvb;
  // Counts come from caller memory: clamp them so that a corrupt BlockMask cannot send the
  // kernel outside the index arrays.
  t.nfull = min(max(a.full_num[row], 0), a.nkvb);
  t.npart = min(max(a.kv_num[row], 0), a.nkvb);
  return t;
}

// Score transform for one accumulator value of query qi and key kv; returns the log2-domain
// logit. SCORE bits: FA_SCORE_ALIBI, FA_SCORE_SOFTCAP (ALiBi first, then the soft-cap). The
// constants are folded on the host: with s = acc * sm_scale - slope * |qi - kv| and
// tanh(x) = 1 - 2 / (1 + e^(2x)), the soft-capped logit in log2 units is
//   C log2(e) - 2 C log2(e) / (1 + 2^(s * 2 log2(e) / C)),
// one multiply (or FMA with ALiBi), exp2, add, reciprocal and FMA per score; `slope` arrives
// pre-multiplied by log2(e) (ALiBi alone) or 2 log2(e) / C (with the soft-cap). exp2 saturates
// to inf or 0 for large |s / C|, giving exactly +-C log2(e).
template <int SCORE>
__device__ __forceinline__ float score_log2(const FwdArgs& a, float acc, int qi, int kv, float slope) {
  if constexpr (SCORE == 0) {
    return acc * a.scale_log2;
  } else if constexpr (SCORE == FA_SCORE_ALIBI) {
    return fmaf(-slope, fabsf((float)(qi - kv)), acc * a.scale_log2);
  } else {
    float u = acc * a.sc_in;
    if constexpr (SCORE & FA_SCORE_ALIBI) u = fmaf(-slope, fabsf((float)(qi - kv)), u);
    return fmaf(a.sc_out2, __builtin_amdgcn_rcpf(1.0f + fast_exp2(u)), a.sc_out);
  }
}

// Soft-cap only: the reciprocal r = 1 / (1 + 2^u) of score_log2, which gives the logit as
// sc_out + sc_out2 * r with sc_out2 < 0. The forward keeps r per score: the logit decreases with
// r, so the row maximum is sc_out + sc_out2 * (row minimum of r), and the exponent argument
// logit - m is one FMA, r * sc_out2 + (sc_out - m). A masked score has r = +inf (logit -inf).
template <int SCORE>
__device__ __forceinline__ float softcap_r(const FwdArgs& a, float acc, int qi, int kv, float slope) {
  float u = acc * a.sc_in;
  if constexpr (SCORE & FA_SCORE_ALIBI) u = fmaf(-slope, fabsf((float)(qi - kv)), u);
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(u));
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// bf16 kernel
//
// A workgroup of WAVES waves (4 or 8) owns 32 * WAVES queries; every wave owns 32. Keys are
// processed in steps of 64 (a 128-key BlockMask tile is two steps). K and V rows of a step live
// in LDS (16 KB each, swizzled 16-byte chunks) in NBUF ring buffers: while one step is
// computed, the next NBUF - 1 steps' K, V and document ids stream into the other buffers with
// global_load_lds_dwordx4, which writes LDS directly without passing through registers. The
// buffers are distinct LDS objects selected at compile time (the step loop is unrolled NBUF
// times): the compiler then knows that reads of one buffer do not depend on the transfers into
// the others and does not wait for them. Every step issues the same fixed number of transfers
// per wave (past the end they re-read row 0 into the buffer just released), so the wait for a
// step's data is one s_waitcnt with a constant count. BlockMask list entries are read 64 at a
// time into one register and picked out with readlane.
//   WAVES = 4, NBUF = 2: 64 KB of LDS, two workgroups per CU (128-query BlockMask blocks);
//   WAVES = 8, NBUF = 4: 128 KB of LDS, one workgroup per CU, three steps in flight
//   (256-query BlockMask blocks; K/V reads are shared by twice the queries).
//
// Mask evaluation (partial tiles only). Causal, window and prefix-LM together allow, for a
// query i, exactly one key interval [lo, hi): causal gives hi = i + 1, prefix-LM gives
// hi = max(prefix_len, i + 1), window gives lo = i - window + 1, and the key count bounds hi.
// Each score therefore needs one unsigned compare, plus one document-id compare under DOC.
// Before any product, each wave drops the 32x32 (query x key) sub-blocks that its mask makes
// entirely empty: their probabilities are exactly 0, so skipping both products changes nothing.
//
// Online softmax with a lazily updated maximum: the running maximum m (log2 units) is raised
// only when a row's new maximum exceeds it by more than kRescaleSlack, so most steps skip the
// O and l rescale. Probabilities exp2(t - m) then stay below 2^kRescaleSlack, far from fp32 and
// bf16 limits, and out = O / l and lse = (m + log2 l) ln 2 are unchanged whichever m is used.
// ---------------------------------------------------------------------------------------------
namespace {

constexpr int kStep = 64;
constexpr int kStepBytes = kStep * 256;
constexpr float kRescaleSlack = 8.0f;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__shared__ __attribute__((aligned(1024))) unsigned char g_k0[kStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char g_v0[kStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char g_k1[kStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char g_v1[kStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char g_k2[kStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char g_v2[kStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char g_k3[kStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char g_v3[kStepBytes];
__shared__ __attribute__((aligned(16))) int g_d0[kStep];
__shared__ __attribute__((aligned(16))) int g_d1[kStep];
__shared__ __attribute__((aligned(16))) int g_d2[kStep];
__shared__ __attribute__((aligned(16))) int g_d3[kStep];

template <int B> __device__ __forceinline__ unsigned char* kbuf() {
  return B == 0 ? g_k0 : B == 1 ? g_k1 : B == 2 ? g_k2 : g_k3;
}
template <int B> __device__ __forceinline__ unsigned char* vbuf() {
  return B == 0 ? g_v0 : B == 1 ? g_v1 : B == 2 ? g_v2 : g_v3;
}
template <int B> __device__ __forceinline__ int* dbuf() { return B == 0 ? g_d0 : B == 1 ? g_d1 : B == 2 ? g_d2 : g_d3; }

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}
// The compiler does not track the LDS writes of global_load_lds; wait for them explicitly:
// at most N vector-memory operations of this wave may still be outstanding.
template <int N> __device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Minimum / maximum over lanes 0..31 (both halves hold the same values where these are used),
// returned wave-uniform. Data-parallel-primitive moves (DPP, a VALU operand modifier, no LDS
// round trip) reduce each 16-lane row: quad_perm swaps of lanes l^1 and l^2, then the
// half-row and row mirrors pair each 4- and 8-lane group with its partner; the two rows are
// then combined in scalar registers.
template <int CTRL> __device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
__device__ __forceinline__ int wave_min32(int x) {
  x = min(x, dpp<kDppXor1>(x));
  x = min(x, dpp<kDppXor2>(x));
  x = min(x, dpp<kDppHalfMirror>(x));
  x = min(x, dpp<kDppMirror>(x));
  return min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
}
__device__ __forceinline__ int wave_max32(int x) {
  x = max(x, dpp<kDppXor1>(x));
  x = max(x, dpp<kDppXor2>(x));
  x = max(x, dpp<kDppHalfMirror>(x));
  x = max(x, dpp<kDppMirror>(x));
  return max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
}

struct StepInfo {
  int kv0;
  bool ok, masked;
};

// Per-lane constants of one workgroup.
struct Ctx {
  int wave, lane, hl, lq, g16, s16;
  int qw0, qw1, qi;
  int hq;                // query head of this lane's row
  bool q_in, doc;
  int qdoc, qd_min, qd_max;
  float slope;
  const __bf16* kp;
  const __bf16* vp;
  const int* kvdoc;      // document ids of this batch, or a valid dummy address without DOC
  int koff, voff;        // element offset of this lane's 16-byte DMA chunk in its first segment
  // Byte offsets within a K or V step buffer of this lane's first operand reads (swizzle
  // applied): kx0 for the K operand of k-step 0 (row lq), vx0 for the transposed V read of
  // channel block 0 at the lane's base row. The other reads follow by XOR (kx_at, vx_at).
  int kx0, vx0;
};

// The swizzle's fields are disjoint bit ranges of the byte offset, so moving to another chunk
// or row block is an XOR. K operand of k-step ks (chunk 2*ks + hl of row lq): the k-step sets
// bits 5-7. Transposed V read of channel block db at base row + 8*j: db sets bits 6-7 of the
// chunk field, and 8 more rows set bit 11 and flip chunk bit 1 (byte bit 5).
__device__ __forceinline__ int kx_at(int kx0, int ks) { return kx0 ^ (32 * ks); }
__device__ __forceinline__ int vx_at(int vx0, int db, int j) { return vx0 ^ (64 * db + 2080 * j); }

struct State {
  f32x16 oacc[4];
  float m_run, l_run;
};

// Transfers of one step: 16 one-KB segments per tensor (4 rows each), WAVES waves issue
// 16 / WAVES of each, plus one transfer of document ids (64 / WAVES per wave). The count per
// wave is therefore the same for every step: 2 * 16 / WAVES + 1.
template <int WAVES> constexpr int step_ops() { return 2 * (16 / WAVES) + 1; }

// Transfer j (0 <= j < 2 * 16 / WAVES) of a step that ends inside the keys: segment j / 2 of K
// (j even) or of V (j odd). Segment i*WAVES + wave holds rows 4*(i*WAVES + wave) + lane/16;
// the chunk swizzle depends on the row modulo 16 only, and segments of one wave differ by
// 4*WAVES rows (a multiple of 16), so they share the lane's chunk offset.
template <int B, int WAVES>
__device__ __forceinline__ void issue_seg(const FwdArgs& a, const Ctx& c, int kv0, int j) {
  const int i = j >> 1;
  const int seg = i * WAVES + c.wave;
  if (j & 1)
    dma16(c.vp + (int64_t)(kv0 + 4 * WAVES * i) * a.v_sl + c.voff, vbuf<B>() + seg * 1024);
  else
    dma16(c.kp + (int64_t)(kv0 + 4 * WAVES * i) * a.k_sl + c.koff, kbuf<B>() + seg * 1024);
}
// The step's document ids (one transfer; a valid dummy address without DOC).
template <int B, int WAVES>
__device__ __forceinline__ void issue_ids(const FwdArgs& a, const Ctx& c, int kv0) {
  constexpr int IDS = kStep / WAVES;  // document ids per wave (lanes 0..IDS-1)
  if (c.lane < IDS) {
    const int* src = c.doc ? c.kvdoc + min(kv0 + c.wave * IDS + c.lane, a.Lkv - 1) : c.kvdoc;
    dma4(src, dbuf<B>() + c.wave * IDS);
  }
}

// All transfers of a step at once. Rows past the end are clamped to the last key: they hold
// finite data and are masked.
template <int B, int WAVES>
__device__ __forceinline__ void issue_step(const FwdArgs& a, const Ctx& c, const StepInfo& si) {
  constexpr int SEGS = 16 / WAVES;  // segments per wave and tensor
  if (si.kv0 + kStep <= a.Lkv) {
#pragma unroll
    for (int j = 0; j < 2 * SEGS; ++j) issue_seg<B, WAVES>(a, c, si.kv0, j);
  } else {
#pragma unroll
    for (int i = 0; i < SEGS; ++i) {
      const int seg = i * WAVES + c.wave;
      const int r = seg * 4 + (c.lane >> 4);
      const int ch = (c.lane & 15) ^ swz(r);
      const int64_t kv = min(si.kv0 + r, a.Lkv - 1);
      dma16(c.kp + kv * a.k_sl + ch * 8, kbuf<B>() + seg * 1024);
      dma16(c.vp + kv * a.v_sl + ch * 8, vbuf<B>() + seg * 1024);
    }
  }
  issue_ids<B, WAVES>(a, c, si.kv0);
}

// MASKED: evaluate the mask per score (partial tiles, ragged last step); DOC: the document
// predicate is part of the mask (a compile-time choice, so that each score costs two compares
// against inline constants, plus one id compare under DOC, and one select).
// ISSUE >= 0: this step also issues the transfers of the next step (which ends inside the keys,
// kv0n) into buffer ISSUE, spread between its S products when both sub-blocks are live (a wave
// is held while its transfers are accepted, and the memory pipeline accepts about 64 bytes per
// cycle per CU, so issuing them back to back stalls every wave of the CU), else up front.
template <int B, int SCORE, bool MASKED, bool DOC, int ISSUE, int WAVES, int MODE>
__device__ __forceinline__ void compute_step(const FwdArgs& a, const Ctx& c, const bf16x8 (&qreg)[8], State& st,
                                             const int kv0, const int kv0n) {
  constexpr int NSEG = 2 * (16 / WAVES);  // row transfers per wave and step
  const unsigned char* sK = kbuf<B>();
  const unsigned char* sV = vbuf<B>();
  const int* sD = dbuf<B>();
  // The offsets are re-defined here (no instruction is emitted) so that the compiler forms
  // buffer + offset inside the loop, where the buffer address folds into the instruction's
  // immediate offset, instead of keeping one hoisted register per buffer and offset.
  int kx0 = c.kx0, vx0 = c.vx0;
  asm volatile("" : "+v"(kx0), "+v"(vx0));
  int dx = 4 * c.hl;  // element offset of this lane's document ids in a step (same reason)
  asm volatile("" : "+v"(dx));
  // This lane's query and its key interval, recomputed per step from the wave's first query
  // (scalar) and the lane's row (kx0 / 256): kept across the loop they would be spilled.
  const int qi = MODE == 2 ? c.qi : c.qw0 + (kx0 >> 8);
  int lo = 0, hi = 0;
  if constexpr (MASKED) key_interval(a, qi, lo, hi);

  // Live 32-key sub-blocks for this wave (wave-uniform).
  unsigned live = 3;
  if constexpr (MASKED) {
    // Document-id range of each sub-block's keys, both at once: lane l reads key l's id (ids
    // past the last key repeat the last key's, which lies in the same sub-block), and each
    // 32-lane half is reduced to its minimum and maximum by DPP moves within 16-lane rows and
    // the two rows' results. lq + 32 hl is the lane: lq is recovered from kx0 (row lq times 256
    // plus a chunk offset below 256), which is live here; c.lq itself would be kept in a spilled
    // register.
    int kd_min[2] = {0, 0}, kd_max[2] = {0, 0};
    if constexpr (DOC) {
      int mx = sD[(kx0 >> 8) + 8 * dx], mn = mx;
      mx = max(mx, dpp<kDppXor1>(mx));
      mn = min(mn, dpp<kDppXor1>(mn));
      mx = max(mx, dpp<kDppXor2>(mx));
      mn = min(mn, dpp<kDppXor2>(mn));
      mx = max(mx, dpp<kDppHalfMirror>(mx));
      mn = min(mn, dpp<kDppHalfMirror>(mn));
      mx = max(mx, dpp<kDppMirror>(mx));
      mn = min(mn, dpp<kDppMirror>(mn));
      kd_max[0] = max(__builtin_amdgcn_readlane(mx, 0), __builtin_amdgcn_readlane(mx, 16));
      kd_max[1] = max(__builtin_amdgcn_readlane(mx, 32), __builtin_amdgcn_readlane(mx, 48));
      kd_min[0] = min(__builtin_amdgcn_readlane(mn, 0), __builtin_amdgcn_readlane(mn, 16));
      kd_min[1] = min(__builtin_amdgcn_readlane(mn, 32), __builtin_amdgcn_readlane(mn, 48));
    }
    live = 0;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int k0 = kv0 + nb * 32;
      if (k0 >= a.Lkv || c.qw0 >= a.Lq) continue;
      const int k1 = min(k0 + 31, a.Lkv - 1);
      bool dead = false;
      if (a.flags & FA_MASK_CAUSAL) dead = dead || c.qw1 < k0;
      if (a.flags & FA_MASK_WINDOW) dead = dead || c.qw0 - k1 >= a.window;
      if (a.flags & FA_MASK_PREFIX_LM) dead = dead || (k0 >= a.prefix_len && c.qw1 < k0);
      if (DOC) dead = dead || (kd_max[nb] < c.qd_min) | (kd_min[nb] > c.qd_max);
      if (!dead) live |= 1u << nb;
    }
    live = __builtin_amdgcn_readfirstlane(live);
  }

  // Everything after the liveness test is straight-line code for a fixed live pattern L (bit nb:
  // sub-block nb is live): a branch per sub-block inside the P.V loop made the compiler keep O
  // in two register sets and copy the accumulators around each branch.
  auto body = [&](auto live_c) {
    constexpr unsigned L = decltype(live_c)::value;
    // S^T = K Q^T for the live 32-key sub-blocks.
    f32x16 sacc[2];
    if constexpr (ISSUE >= 0 && L == 3u) {
      // Both sub-blocks: the two product chains alternate, and one transfer of the next step
      // follows each pair of products.
      issue_ids<(ISSUE < 0 ? 0 : ISSUE), WAVES>(a, c, kv0n);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const bf16x8 kf = *(const bf16x8*)(sK + nb * 32 * 256 + kx_at(kx0, ks));
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[ks], ks ? sacc[nb] : f32x16{}, 0, 0, 0);
        }
        if (ks < NSEG) issue_seg<(ISSUE < 0 ? 0 : ISSUE), WAVES>(a, c, kv0n, ks);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ks < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ks < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (ks < NSEG) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    } else {
      if constexpr (ISSUE >= 0) {
        StepInfo nx{kv0n, true, false};
        issue_step<ISSUE, WAVES>(a, c, nx);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (!(L & (1u << nb))) continue;
        sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(sK + nb * 32 * 256 + kx0), qreg[0],
                                                           f32x16{}, 0, 0, 0);
#pragma unroll
        for (int ks = 1; ks < 8; ++ks) {
          const bf16x8 kf = *(const bf16x8*)(sK + nb * 32 * 256 + kx_at(kx0, ks));
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[ks], sacc[nb], 0, 0, 0);
        }
        // Schedule: 4 operand reads ahead, then one read per product (bounds live operands).
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (k < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }

    // Scores (log2 domain) and the mask. Without a score_mod the 1/sqrt(d) * log2(e) scale is
    // folded into the exponent below, and the maximum is taken on the raw products. With the
    // soft-cap the tile keeps r (see softcap_r) and the row minimum of r gives the maximum.
    constexpr bool CAP = (SCORE & FA_SCORE_SOFTCAP) != 0;
    float mx = CAP ? INFINITY : -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (!(L & (1u << nb))) continue;
      const int kbase = kv0 + nb * 32 + c.hl * 4;   // key of element i is kbase + (i/4)*8 + i%4
      // The allowed keys [lo, hi) relative to kbase: element offsets are the constants 0..27.
      // They become one bitmask per lane (bit off set: offset off allowed); each score then
      // takes its bit with a signed bitfield extract (0 or all ones) and keeps its bits or
      // those of -inf with a bitfield insert: two vector operations and no lane masks.
      unsigned abits = 0;
      if constexpr (MASKED) {
        const int l0 = min(max(lo - kbase, 0), 31), h0 = min(max(hi - kbase, 0), 31);
        abits = ((1u << h0) - 1u) & ~((1u << l0) - 1u);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        i32x4 kd4 = i32x4{};
        if constexpr (MASKED && DOC) kd4 = *(const i32x4*)(sD + dx + nb * 32 + g * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = g * 4 + e;
          const int off = g * 8 + e;
          float x = SCORE == 0 ? sacc[nb][i]
                    : CAP         ? softcap_r<SCORE>(a, sacc[nb][i], qi, kbase + off, c.slope)
                                  : score_log2<SCORE>(a, sacc[nb][i], qi, kbase + off, c.slope);
          if constexpr (MASKED) {
            constexpr unsigned kMasked = CAP ? 0x7f800000u : 0xff800000u;  // +inf (r) or -inf
            const int keep = (int)(abits << (31 - off)) >> 31;
            x = __int_as_float((__float_as_int(x) & keep) | (int)(kMasked & ~(unsigned)keep));
            if constexpr (DOC) x = kd4[e] == c.qdoc ? x : __uint_as_float(kMasked);
          }
          sacc[nb][i] = x;
          mx = CAP ? fminf(mx, x) : fmaxf(mx, x);
        }
      }
    }
    mx = CAP ? fmaf(a.sc_out2, half_swap_min(mx), a.sc_out) : half_swap_max(mx);
    const float scale = SCORE == 0 ? a.scale_log2 : 1.0f;
    const float m_cand = fmaxf(st.m_run, mx * scale);
    const bool raise = m_cand > st.m_run + kRescaleSlack;

    // The exponentials and P.V products follow in two copies, one per outcome of the rescale
    // test: with one copy after a conditional rescale, the compiler kept O in two register sets
    // and copied all 64 accumulators on every step.
    auto finish = [&]() {
      const float m_eff = st.m_run == -INFINITY ? 0.f : st.m_run;  // rows with no allowed key so far
      const float cap_off = a.sc_out - m_eff;
      // P = exp2(t - m); P^T goes straight into the B operand of O^T = V^T P^T as bf16.
      bf16x8 pb[2][2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (!(L & (1u << nb))) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(CAP ? fmaf(sacc[nb][i], a.sc_out2, cap_off) : fmaf(sacc[nb][i], scale, -m_eff));
          st.l_run += p;
          pb[nb][i >> 3][i & 7] = (__bf16)p;
        }
      }
      // O^T += V^T P^T. A operand (V^T: row = channel, k = key) by transposed LDS reads: in each
      // 16-lane group, source lane s points at key row base + s/4 and channels d0 + 4*(s%4);
      // lane i of the group then receives V[base + j][d0 + i], j = 0..3.
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if (!(L & (1u << nb))) continue;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int rows = (nb * 32 + h * 16) * 256;  // the swizzle depends on the row modulo 16
            const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sV + rows + vx_at(vx0, db, 0)));
            const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sV + rows + vx_at(vx0, db, 1)));
            // Whole-vector concatenation and bit cast (element-wise bf16 inserts of the i16 lanes
            // were observed to be folded into a broadcast of element 0).
            const i16x8 cat = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            st.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pb[nb][h],
                                                                  st.oacc[db], 0, 0, 0);
          }
        }
        if constexpr (L == 3u) {
          // Schedule: 4 transposed reads ahead, then two reads per product.
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            if (k < 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
          }
        }
      }
    };
    if (__builtin_amdgcn_readfirstlane(__ballot(raise) != 0)) {
      // Rows that keep m (including rows still at -inf) must get alpha = 1 exactly; a raised row
      // coming from -inf gets exp2(-inf) = 0.
      const float m_new = raise ? m_cand : st.m_run;
      const float alpha = raise ? fast_exp2(st.m_run - m_new) : 1.0f;
      st.l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) st.oacc[db] *= alpha;
      st.m_run = m_new;
      finish();
    } else {
      finish();
    }
  };

  if constexpr (!MASKED) {
    if (MODE > 0 && c.qw0 >= a.Lq) {
      // A wave past the last query (few query rows, as in decoding) only does its share of the
      // transfers; its products would be discarded. (Masked steps find this in the liveness test.)
      if constexpr (ISSUE >= 0) {
        StepInfo nx{kv0n, true, false};
        issue_step<ISSUE, WAVES>(a, c, nx);
      }
      return;
    }
    body(std::integral_constant<unsigned, 3u>{});
  } else {
    if (live == 0u) {
      if constexpr (ISSUE >= 0) {
        StepInfo nx{kv0n, true, false};
        issue_step<ISSUE, WAVES>(a, c, nx);
      }
      return;
    }
    if (live == 3u) body(std::integral_constant<unsigned, 3u>{});
    else if (live == 1u) body(std::integral_constant<unsigned, 1u>{});
    else body(std::integral_constant<unsigned, 2u>{});
  }
}

}  // namespace

// MODE > 0: the split-KV form (a range of each tile list, partial results; waves without a
// query skip the products); MODE 2 also packs the query heads of one kv head (see decode_work).
// Separate instantiations, so that the plain forward carries none of it.
template <int TB, int SCORE, int WAVES, int NBUF, int MODE>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int HALVES = TB / kStep;
  constexpr int BQ = 32 * WAVES;
  constexpr int OPS = step_ops<WAVES>();

  const WorkItem it = decode_work<MODE>(a, blockIdx.x);
  Ctx c;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar registers
  c.lane = threadIdx.x & 63;
  c.hl = c.lane >> 5;
  c.lq = c.lane & 31;
  c.g16 = c.lane >> 4;
  c.s16 = c.lane & 15;
  if constexpr (MODE == 2) {
    // Row r = 32 * wave + lq holds query r % Lq of head r / Lq of the group (group * Lq <= 128).
    const int r = c.wave * 32 + c.lq;
    const int g = r / a.Lq;
    c.qi = r - g * a.Lq;
    c.q_in = g < a.group;
    c.hq = it.hkv * a.group + min(g, a.group - 1);
    c.qw0 = wave_min32(c.q_in ? c.qi : INT_MAX);  // INT_MAX: the wave holds no row
    c.qw1 = wave_max32(c.q_in ? c.qi : INT_MIN);
  } else {
    c.qw0 = it.qb * BQ + c.wave * 32;
    c.qw1 = min(c.qw0 + 31, a.Lq - 1);
    c.qi = c.qw0 + c.lq;
    c.q_in = c.qi < a.Lq;
    c.hq = it.hq;
  }
  c.doc = (a.flags & FA_MASK_DOC) != 0;
  c.kp = (const __bf16*)a.k + it.b * a.k_sb + it.hkv * a.k_sh;
  c.vp = (const __bf16*)a.v + it.b * a.v_sb + it.hkv * a.v_sh;
  c.kvdoc = c.doc ? a.kv_doc + (int64_t)it.b * a.Lkv : (const int*)c.kp;
  c.kx0 = tile_off(c.lq, c.hl);
  {
    // In each 16-lane group, source lane s points at key row base + s/4, channels d0 + 4*(s%4).
    const int d = 16 * (c.g16 & 1) + 4 * (c.s16 & 3);
    const int r0 = (c.g16 >> 1) * 4 + (c.s16 >> 2);
    c.vx0 = tile_off(r0, d >> 3) + (d & 7) * 2;
  }
  {
    const int r = c.wave * 4 + (c.lane >> 4);  // row of this lane in its first segment
    const int ch = (c.lane & 15) ^ swz(r);
    c.koff = r * (int)a.k_sl + ch * 8;
    c.voff = r * (int)a.v_sl + ch * 8;
  }

  int chunk_init;
  // First-round loads, all issued before any of them is waited for (one memory round trip):
  // this lane's Q row, its document id, the BlockMask counts and the first 64 entries of both
  // index lists (the index rows always hold n_kvb entries, so no count is needed to read them).
  // Addresses are clamped or redirected to valid memory instead of branching around the loads;
  // the values are discarded afterwards where they do not apply.
  // Q^T as the B operand: lane holds Q[qi][16*ks + 8*hl .. +8] for ks = 0..7.
  const __bf16* qp = (const __bf16*)a.q + it.b * a.q_sb + c.hq * a.q_sh;
  const int qi_c = min(c.qi, a.Lq - 1);
  bf16x8 qreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qreg[ks] = *(const bf16x8*)(qp + (int64_t)qi_c * a.q_sl + ks * 16 + c.hl * 8);
  const int* qdoc_p = c.doc ? a.q_doc + (int64_t)it.b * a.Lq + qi_c : (const int*)qp;
  const int qdoc_raw = *qdoc_p;
  TileList tl;
  {
    const int bm = a.Bm == 1 ? 0 : it.b;
    const int hm = a.Hm == 1 ? 0 : it.hq;
    const int64_t row = ((int64_t)bm * a.Hm + hm) * a.nqb + it.qb;
    // Without a BlockMask the list pointers are null, and with no key block (n_kvb = 0) the
    // index rows are empty: the list reads then go to this head's first Q row (256 bytes, 64
    // ints, always present when a workgroup runs) and are ignored.
    const int* dummy = (const int*)((const __bf16*)a.q + it.b * a.q_sb + it.hq * a.q_sh);
    const bool no_lists = a.all_full || a.nkvb == 0;
    tl.full = no_lists ? dummy : a.full_idx + row * a.nkvb;
    tl.part = no_lists ? dummy : a.kv_idx + row * a.nkvb;
    const int fn = *(a.all_full ? dummy : a.full_num + row);
    const int pn = *(a.all_full ? dummy : a.kv_num + row);
    const int lc = max(min(c.lane, a.nkvb - 1), 0);  // in [0, 63] and inside the row
    const int fch = tl.full[lc];
    const int pch = tl.part[lc];
    // Counts come from caller memory: clamp them so that a corrupt BlockMask cannot send the
    // kernel outside the index arrays.
    tl.nfull = a.all_full ? a.nkvb : min(max(fn, 0), a.nkvb);
    tl.npart = a.all_full ? 0 : min(max(pn, 0), a.nkvb);
    // Merge: entries of the full list, then of the partial list, with one cross-lane move.
    const int pmv = __shfl(pch, (c.lane - tl.nfull) & 63, 64);
    chunk_init = c.lane < tl.nfull ? fch : pmv;
  }
  if (!c.q_in) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = bf16x8{};
  }
  c.qdoc = (c.doc && c.q_in) ? qdoc_raw : 0;
  const int ntiles = tl.nfull + tl.npart;
  // Split-KV: this workgroup takes list entries [t_begin, t_end).
  int t_begin = 0, t_end = ntiles;
  if constexpr (MODE > 0) {
    t_begin = (int)((int64_t)it.split * ntiles / a.nsplit);
    t_end = (int)((int64_t)(it.split + 1) * ntiles / a.nsplit);
  }
  const int nsteps = (t_end - t_begin) * HALVES;

  // List entries, 64 per register: lane j holds the entry of tile chunk_base + j.
  auto load_chunk = [&](int base) -> int {
    const int t = base + c.lane;
    if (a.all_full || t >= ntiles) return t;
    return t < tl.nfull ? tl.full[t] : tl.part[t - tl.nfull];
  };
  int chunk_base = 0;
  int chunk = chunk_init;
  c.slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[c.hq] * a.slope_mul : 0.f;

  // Step s -> StepInfo (steps past the end re-read row 0 and are not computed).
  auto info = [&](int s) {
    StepInfo si{0, false, false};
    if (s >= nsteps) return si;
    const int t = t_begin + s / HALVES;
    if (t >= chunk_base + 64) {  // next 64 list entries (once per 64 tiles)
      chunk_base = t & ~63;
      chunk = load_chunk(chunk_base);
    }
    const int kb = a.all_full ? t : __builtin_amdgcn_readlane(chunk, t - chunk_base);
    // A corrupt index is skipped rather than read out of range; so is a half past the end.
    const int kv0 = kb * TB + (s % HALVES) * kStep;
    si.ok = kb >= 0 && kb < a.nkvb && kv0 < a.Lkv;
    si.kv0 = si.ok ? kv0 : 0;
    si.masked = (t >= tl.nfull) || (kv0 + kStep > a.Lkv);
    return si;
  };

  State st;
#pragma unroll
  for (int db = 0; db < 4; ++db) st.oacc[db] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  // Prologue: steps 0 .. NBUF-2 in flight. Without any step (no key, or an empty BlockMask
  // row) nothing is transferred at all: the padding transfers below need one valid key row.
  StepInfo ring[NBUF];
  if (nsteps > 0) {
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j) {
      ring[j] = info(j);
      if (j == 0) issue_step<0, WAVES>(a, c, ring[j]);
      if (j == 1) issue_step<1, WAVES>(a, c, ring[j]);
      if (j == 2) issue_step<2, WAVES>(a, c, ring[j]);
    }
  }
  c.qd_min = c.qd_max = 0;
  if (c.doc) {
    c.qd_min = wave_min32(c.q_in ? c.qdoc : INT_MAX);
    c.qd_max = wave_max32(c.q_in ? c.qdoc : INT_MIN);
  }

  // One step: wait for its transfers (NBUF-2 later steps may stay in flight), make sure every
  // wave is done with the buffer about to be refilled, refill it with step s + NBUF - 1, compute.
  auto step = [&](auto bufc, int s) {
    constexpr int B = decltype(bufc)::value;
    constexpr int NB = (B + NBUF - 1) % NBUF;
    wait_vmem<(NBUF - 2) * OPS>();
    __syncthreads();
    const StepInfo nxt = info(s + NBUF - 1);
    const StepInfo cur = ring[B];
    ring[NB] = nxt;
    if (cur.ok && nxt.kv0 + kStep <= a.Lkv) {
      // The step's own compute issues the next step's transfers.
      if (!cur.masked) compute_step<B, SCORE, false, false, NB, WAVES, MODE>(a, c, qreg, st, cur.kv0, nxt.kv0);
      else if (c.doc) compute_step<B, SCORE, true, true, NB, WAVES, MODE>(a, c, qreg, st, cur.kv0, nxt.kv0);
      else compute_step<B, SCORE, true, false, NB, WAVES, MODE>(a, c, qreg, st, cur.kv0, nxt.kv0);
    } else {
      issue_step<NB, WAVES>(a, c, nxt);
      if (cur.ok) {
        if (!cur.masked) compute_step<B, SCORE, false, false, -1, WAVES, MODE>(a, c, qreg, st, cur.kv0, 0);
        else if (c.doc) compute_step<B, SCORE, true, true, -1, WAVES, MODE>(a, c, qreg, st, cur.kv0, 0);
        else compute_step<B, SCORE, true, false, -1, WAVES, MODE>(a, c, qreg, st, cur.kv0, 0);
      }
    }
  };
  for (int s = 0; s < nsteps; s += NBUF) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 < nsteps) step(std::integral_constant<int, 1 % NBUF>{}, s + 1);
    if constexpr (NBUF > 2) {
      if (s + 2 < nsteps) step(std::integral_constant<int, 2 % NBUF>{}, s + 2);
      if (s + 3 < nsteps) step(std::integral_constant<int, 3 % NBUF>{}, s + 3);
    }
  }
  wait_vmem<0>();  // no transfer may outlive the workgroup's LDS

  // Epilogue: combine the two halves' row sums, normalise, store O (bf16) and the natural-log lse.
  const float l_tot = half_swap_sum(st.l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if constexpr (MODE > 0) {
    // Split-KV partial result: normalised O in fp32 and the lse of this range of tiles.
    if (c.q_in) {
      const int64_t prow = (((int64_t)it.split * a.B + it.b) * a.Hq + c.hq) * a.Lq + c.qi;
      float* po = a.part_o + prow * 128;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = st.oacc[db][gq * 4 + e] * inv;
          *(f32x4*)(po + db * 32 + gq * 8 + c.hl * 4) = o4;
        }
      }
      if (c.hl == 0) a.part_lse[prow] = l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  if constexpr (WAVES == 4) {
    // O goes out through LDS, so that each store writes whole rows: in registers a lane holds 4
    // channels of each of 16 channel groups of its row, and stored from there every instruction
    // wrote 16 bytes into each of 32 rows. Waves 0-1 stage their 32 x 256-byte rows in the first
    // K buffer, waves 2-3 in the first V buffer (free once every wave is past its last step), in
    // the swizzled tile layout; each wave reads back only its own rows.
    __syncthreads();
    unsigned char* const ob = (c.wave < 2 ? kbuf<0>() : vbuf<0>()) + (c.wave & 1) * (32 * 256);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 o4;
        o4[0] = (__bf16)(st.oacc[db][gq * 4 + 0] * inv);
        o4[1] = (__bf16)(st.oacc[db][gq * 4 + 1] * inv);
        o4[2] = (__bf16)(st.oacc[db][gq * 4 + 2] * inv);
        o4[3] = (__bf16)(st.oacc[db][gq * 4 + 3] * inv);
        *(bf16x4*)(ob + tile_off(c.lq, db * 4 + gq) + c.hl * 8) = o4;
      }
    }
    // Row r of the wave (4 rows per instruction), 16-byte chunk lane % 16.
    __bf16* const op0 = (__bf16*)a.o + it.b * a.o_sb + it.hq * a.o_sh;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (c.lane >> 4), ch = c.lane & 15;
      const bf16x8 v8 = *(const bf16x8*)(ob + tile_off(r, ch));
      const int q = c.qw0 + r;
      if (q < a.Lq) *(bf16x8*)(op0 + (int64_t)q * a.o_sl + ch * 8) = v8;
    }
    if (c.q_in && a.lse && c.hl == 0) {
      a.lse[((int64_t)it.b * a.Hq + it.hq) * a.Lq + c.qi] =
          l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  if (c.q_in) {
    __bf16* op = (__bf16*)a.o + it.b * a.o_sb + it.hq * a.o_sh + (int64_t)c.qi * a.o_sl;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 o4;
        o4[0] = (__bf16)(st.oacc[db][gq * 4 + 0] * inv);
        o4[1] = (__bf16)(st.oacc[db][gq * 4 + 1] * inv);
        o4[2] = (__bf16)(st.oacc[db][gq * 4 + 2] * inv);
        o4[3] = (__bf16)(st.oacc[db][gq * 4 + 3] * inv);
        *(bf16x4*)(op + db * 32 + gq * 8 + c.hl * 4) = o4;
      }
    }
    if (a.lse && c.hl == 0) {
      a.lse[((int64_t)it.b * a.Hq + it.hq) * a.Lq + c.qi] =
          l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// One BK-key tile of K and V (fp32) into LDS rows of P floats, 256 threads. Every load of a
// thread is issued before any is waited for, so a tile costs one memory round trip (a rolled
// loop waited for each of its 16 pairs of loads in turn). Rows past the last key are zero; their
// loads read the last key's row instead.
template <int BK, int P>
__device__ __forceinline__ void stage_f32_tile(const FwdArgs& a, const float* kp, const float* vp, int kv0, int tid,
                                               float* sK, float* sV) {
  constexpr int IT = BK * 32 / 256;  // float4 chunks per thread and tensor
  f32x4 kx[IT], vx[IT];
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const int id = tid + j * 256;
    const int64_t kv = min(kv0 + (id >> 5), a.Lkv - 1);
    kx[j] = *(const f32x4*)(kp + kv * a.k_sl + (id & 31) * 4);
    vx[j] = *(const f32x4*)(vp + kv * a.v_sl + (id & 31) * 4);
  }
#pragma unroll
  for (int j = 0; j < IT; ++j) {
    const int id = tid + j * 256;
    const int r = id >> 5, c4 = id & 31;
    const bool in = kv0 + r < a.Lkv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sK[r * P + c4 * 4 + e] = in ? kx[j][e] : 0.f;
      sV[r * P + c4 * 4 + e] = in ? vx[j][e] : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// f32 kernel: same decomposition with v_mfma_f32_32x32x2_f32 (true fp32 products and sums).
// The MFMA's two k positions per instruction are the lane halves; for S^T the k index is the
// channel d = 2*ks + hl, for O^T it is the key of accumulator element i.
// ---------------------------------------------------------------------------------------------
template <int BK, int SCORE>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(FwdArgs a) {
  constexpr int NB = BK / 32;
  constexpr int P = 130;  // LDS row pitch in floats: 2*r + d spreads 64 lanes over 64 banks
  __shared__ float sK[BK * P];
  __shared__ float sV[BK * P];
  __shared__ int sDoc[BK];

  const WorkItem it = decode_work(a, blockIdx.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, lq = lane & 31;
  const int qi = it.qb * kBQ + wave * 32 + lq;
  const bool q_in = qi < a.Lq;

  const float* qp = (const float*)a.q + it.b * a.q_sb + it.hq * a.q_sh;
  const float* kp = (const float*)a.k + it.b * a.k_sb + it.hkv * a.k_sh;
  const float* vp = (const float*)a.v + it.b * a.v_sb + it.hkv * a.v_sh;

  float qreg[64];
#pragma unroll
  for (int ks = 0; ks < 64; ++ks) qreg[ks] = q_in ? qp[(int64_t)qi * a.q_sl + 2 * ks + hl] : 0.f;
  const int qdoc = ((a.flags & FA_MASK_DOC) && q_in) ? a.q_doc[(int64_t)it.b * a.Lq + qi] : 0;
  const float slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[it.hq] * a.slope_mul : 0.f;
  const MaskSpec ms{a.flags, a.window, a.prefix_len};

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const TileList tl = tile_list(a, it);
  const int ntiles = tl.nfull + tl.npart;
  for (int t = 0; t < ntiles; ++t) {
    const bool partial = t >= tl.nfull;
    const int kb = partial ? tl.part[t - tl.nfull] : (a.all_full ? t : tl.full[t]);
    if (kb < 0 || kb >= a.nkvb) continue;
    const int kv0 = kb * BK;
    const bool masked = partial || (kv0 + BK > a.Lkv);

    __syncthreads();
    // The tile's document ids are loaded with K and V (same round trip).
    const bool tile_doc = masked && (a.flags & FA_MASK_DOC) && tid < BK;
    const int kdoc = tile_doc ? a.kv_doc[(int64_t)it.b * a.Lkv + min(kv0 + tid, a.Lkv - 1)] : 0;
    stage_f32_tile<BK, P>(a, kp, vp, kv0, tid, sK, sV);
    if (tile_doc) sDoc[tid] = kv0 + tid < a.Lkv ? kdoc : 0;
    __syncthreads();

    f32x16 sacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      sacc[nb] = f32x16{};
      const float* krow = sK + (nb * 32 + lq) * P + hl;
#pragma unroll
      for (int ks = 0; ks < 64; ++ks)
        sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * ks], qreg[ks], sacc[nb], 0, 0, 0);
    }

    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kv = kv0 + nb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
        float x = score_log2<SCORE>(a, sacc[nb][i], qi, kv, slope);
        if (masked) {
          const int kvdoc = (a.flags & FA_MASK_DOC) ? sDoc[kv - kv0] : 0;
          const bool keep = kv < a.Lkv && mask_pair(ms, qi, kv, qdoc, kvdoc);
          x = keep ? x : -INFINITY;
        }
        sacc[nb][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(sacc[nb][i] - m_use);
        rs += p;
        sacc[nb][i] = p;
      }
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = nb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[r * P + db * 32 + lq], sacc[nb][i], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  const float l_tot = half_swap_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_in) {
    float* op = (float*)a.o + it.b * a.o_sb + it.hq * a.o_sh + (int64_t)qi * a.o_sl;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 o4;
        o4[0] = oacc[db][gq * 4 + 0] * inv;
        o4[1] = oacc[db][gq * 4 + 1] * inv;
        o4[2] = oacc[db][gq * 4 + 2] * inv;
        o4[3] = oacc[db][gq * 4 + 3] * inv;
        *(f32x4*)(op + db * 32 + gq * 8 + hl * 4) = o4;
      }
    }
    if (a.lse && hl == 0) {
      a.lse[((int64_t)it.b * a.Hq + it.hq) * a.Lq + qi] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// fp32 work items below which the split-key kernel runs (one work item per CU or fewer).
constexpr int kF32SplitBelow = 256;

// ---------------------------------------------------------------------------------------------
// f32 split-key kernel, for inputs too small to fill the GPU (a few hundred queries per head, as
// in the grouped-variate layer): the four workgroups of one work item take 32 queries each, and
// the four waves of a workgroup share those queries and take one 32-key sub-block each of every
// tile (sub-blocks nb = wave, wave + 4, ...). Each wave keeps its own online-softmax state; at the
// end the partial results are merged in a fixed wave order through LDS:
//   m = max_w m_w,  f_w = 2^(m_w - m),  l = sum_w f_w l_w,  O = (sum_w f_w O_w) / l.
// A wave reads each K/V sub-block once, so a tile costs each wave a quarter of the products.
//
// Latency is what matters at these sizes, so every phase is one round trip or one barrier:
//   - the workgroup's 32 Q rows are loaded once, coalesced, with the first tile's K and V, and
//     handed to the waves through LDS (per-lane loads of the Q^T operand, 64 four-byte loads per
//     lane, took a third of the kernel);
//   - tile rows past the last key are not loaded;
//   - the four P.V product chains (one per 32-channel block) are interleaved, and S^T is summed
//     in two interleaved chains;
//   - the merge writes each wave's scaled partial O into its own LDS slab and sums the slabs in
//     wave order after a single barrier.
// ---------------------------------------------------------------------------------------------
template <int BK>
struct F32Tile {
  static constexpr int IT = BK * 32 / 256;  // float4 chunks per thread and tensor
  f32x4 k[IT], v[IT];
};

// Loads of one BK-key tile (rows past the last key are skipped).
template <int BK>
__device__ __forceinline__ void f32_tile_load(F32Tile<BK>& tt, const FwdArgs& a, const float* kp, const float* vp,
                                              int kv0, int tid) {
#pragma unroll
  for (int j = 0; j < F32Tile<BK>::IT; ++j) {
    const int id = tid + j * 256;
    const int kv = kv0 + (id >> 5);
    tt.k[j] = f32x4{};
    tt.v[j] = f32x4{};
    if (kv < a.Lkv) {
      tt.k[j] = *(const f32x4*)(kp + (int64_t)kv * a.k_sl + (id & 31) * 4);
      tt.v[j] = *(const f32x4*)(vp + (int64_t)kv * a.v_sl + (id & 31) * 4);
    }
  }
}

template <int BK, int P>
__device__ __forceinline__ void f32_tile_store(const F32Tile<BK>& tt, float* sK, float* sV, int tid) {
#pragma unroll
  for (int j = 0; j < F32Tile<BK>::IT; ++j) {
    const int id = tid + j * 256;
    const int r = id >> 5, c4 = id & 31;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sK[r * P + c4 * 4 + e] = tt.k[j][e];
      sV[r * P + c4 * 4 + e] = tt.v[j][e];
    }
  }
}

template <int BK, int SCORE>
__global__ __launch_bounds__(256, 1) void fwd_f32_split_kernel(FwdArgs a) {
  constexpr int NB = BK / 32;
  constexpr int P = 130;   // K/V/Q row stride in floats
  constexpr int PO = 132;  // merge slab row stride (16-byte rows)
  constexpr int KV_FLOATS = BK * P > 2 * 32 * PO ? BK * P : 2 * 32 * PO;  // a tile, or two merge slabs
  __shared__ __attribute__((aligned(16))) float sK[KV_FLOATS];
  __shared__ __attribute__((aligned(16))) float sV[KV_FLOATS];
  __shared__ float sQ[32 * P];
  __shared__ __attribute__((aligned(16))) int sDoc[BK];
  __shared__ float s_m[4][32];
  __shared__ float s_l[4][32];

  const WorkItem it = decode_work(a, blockIdx.x >> 2);
  const int sub = blockIdx.x & 3;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, lq = lane & 31;
  const int q0 = it.qb * kBQ + sub * 32;
  if (q0 >= a.Lq) return;  // the whole workgroup: no query in this 32-row slice
  const int qi = q0 + lq;
  const bool q_in = qi < a.Lq;

  const float* qp = (const float*)a.q + it.b * a.q_sb + it.hq * a.q_sh;
  const float* kp = (const float*)a.k + it.b * a.k_sb + it.hkv * a.k_sh;
  const float* vp = (const float*)a.v + it.b * a.v_sb + it.hkv * a.v_sh;

  // The slice's Q rows, coalesced: 32 rows x 32 float4 chunks, 4 per thread (rows past the last
  // query are zero).
  f32x4 qst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int id = tid + j * 256;
    const int r = q0 + (id >> 5);
    qst[j] = f32x4{};
    if (r < a.Lq) qst[j] = *(const f32x4*)(qp + (int64_t)r * a.q_sl + (id & 31) * 4);
  }
  const int qdoc = ((a.flags & FA_MASK_DOC) && q_in) ? a.q_doc[(int64_t)it.b * a.Lq + qi] : 0;
  const float slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[it.hq] * a.slope_mul : 0.f;
  // This lane's allowed key interval [klo, khi) under the index predicates and the key count.
  int klo, khi;
  key_interval(a, qi, klo, khi);
  const bool docm = (a.flags & FA_MASK_DOC) != 0;

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  float qreg[64];

  const TileList tl = tile_list(a, it);
  const int ntiles = tl.nfull + tl.npart;
  bool q_staged = false;
  for (int t = 0; t < ntiles; ++t) {
    const bool partial = t >= tl.nfull;
    const int kb = partial ? tl.part[t - tl.nfull] : (a.all_full ? t : tl.full[t]);
    if (kb < 0 || kb >= a.nkvb) continue;
    const int kv0 = kb * BK;
    const bool masked = partial || (kv0 + BK > a.Lkv);

    // The tile's K, V and document ids are loaded in one round trip (with Q, for the first).
    const bool tile_doc = masked && (a.flags & FA_MASK_DOC) && tid < BK;
    const int kdoc = tile_doc ? a.kv_doc[(int64_t)it.b * a.Lkv + min(kv0 + tid, a.Lkv - 1)] : 0;
    F32Tile<BK> tt;
    f32_tile_load<BK>(tt, a, kp, vp, kv0, tid);
    __syncthreads();  // the previous tile's reads are done
    if (!q_staged) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int id = tid + j * 256;
#pragma unroll
        for (int e = 0; e < 4; ++e) sQ[(id >> 5) * P + (id & 31) * 4 + e] = qst[j][e];
      }
    }
    f32_tile_store<BK, P>(tt, sK, sV, tid);
    if (tile_doc) sDoc[tid] = kv0 + tid < a.Lkv ? kdoc : 0;
    __syncthreads();
    if (!q_staged) {
      // Q^T as the B operand: lane holds Q[qi][2 ks + hl].
#pragma unroll
      for (int ks = 0; ks < 64; ++ks) qreg[ks] = sQ[lq * P + 2 * ks + hl];
      q_staged = true;
    }

    for (int nb = wave; nb < NB; nb += 4) {
      if (kv0 + nb * 32 >= a.Lkv) break;  // this and later sub-blocks lie past the last key
      // S^T in two interleaved chains (even and odd k-steps), summed at the end. All 64 K operands
      // are read before the chain (read next to each product, every pair waited for its read).
      float kf[64];
      const float* krow = sK + (nb * 32 + lq) * P + hl;
#pragma unroll
      for (int ks = 0; ks < 64; ++ks) kf[ks] = krow[2 * ks];
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 64; ks += 2) {
        s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[ks], qreg[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[ks + 1], qreg[ks + 1], s1, 0, 0, 0);
      }
      f32x16 sacc = s0 + s1;
      // The 64 V operands of this sub-block, read while the softmax below runs.
      float vf[64];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = nb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
#pragma unroll
        for (int db = 0; db < 4; ++db) vf[i * 4 + db] = sV[r * P + db * 32 + lq];
      }

      // Mask without branches: the key interval and, under DOC, the ids of 4 keys per LDS read.
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const i32x4 kd4 = *(const i32x4*)(sDoc + nb * 32 + g * 8 + hl * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          const int kv = kv0 + nb * 32 + g * 8 + hl * 4 + e;
          float x = score_log2<SCORE>(a, sacc[i], qi, kv, slope);
          const bool keep = !masked | ((kv >= klo) & (kv < khi) & (!docm | (kd4[e] == qdoc)));
          x = keep ? x : -INFINITY;
          sacc[i] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(sacc[i] - m_use);
        rs += p;
        sacc[i] = p;
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      // O^T += V^T P^T, the four channel blocks' chains interleaved.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[i * 4 + db], sacc[i], oacc[db], 0, 0, 0);
      }
    }
  }

  // Merge of the four waves' partial results, in wave order (deterministic).
  const float l_w = half_swap_sum(l_run);
  __syncthreads();  // every wave is done with sK / sV
  if (hl == 0) {
    s_m[wave][lq] = m_run;
    s_l[wave][lq] = l_w;
  }
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) m = fmaxf(m, s_m[w][lq]);
  float l = 0.f, f_self = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = s_m[w][lq];
    const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - m);
    l += f * s_l[w][lq];
    if (w == wave) f_self = f;
  }
  // Slab of wave w: [32 queries][PO], in sK (waves 0, 1) or sV (waves 2, 3). Lane (lq, hl) holds
  // channels 32 db + 8 gq + 4 hl + 0..3 of its query.
  float* slab = (wave < 2 ? sK : sV) + (wave & 1) * 32 * PO;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      f32x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = oacc[db][gq * 4 + e] * f_self;
      *(f32x4*)(slab + lq * PO + db * 32 + gq * 8 + hl * 4) = o4;
    }
  }
  __syncthreads();
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  // Store: wave w writes channels [32 w, 32 w + 32) of the 32 rows (lane = row, two halves of 16),
  // each the sum of the four slabs in wave order.
  if (q_in) {
    float* op = (float*)a.o + it.b * a.o_sb + it.hq * a.o_sh + (int64_t)qi * a.o_sl;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int ch = wave * 32 + hl * 16 + c4 * 4;
      const f32x4 v0 = *(const f32x4*)(sK + lq * PO + ch);
      const f32x4 v1 = *(const f32x4*)(sK + 32 * PO + lq * PO + ch);
      const f32x4 v2 = *(const f32x4*)(sV + lq * PO + ch);
      const f32x4 v3 = *(const f32x4*)(sV + 32 * PO + lq * PO + ch);
      f32x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (((v0[e] + v1[e]) + v2[e]) + v3[e]) * inv;
      *(f32x4*)(op + ch) = o4;
    }
    if (a.lse && wave == 0 && hl == 0) {
      a.lse[((int64_t)it.b * a.Hq + it.hq) * a.Lq + qi] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <int BK, int SCORE>
static hipError_t launch_t(const FwdArgs& a, int dtype, int q_block, hipStream_t stream) {
  if (dtype == 1) {
    if (q_block == 256)
      hipLaunchKernelGGL((fwd_bf16_kernel<BK, SCORE, 8, 4, 0>), dim3(a.total_wg), dim3(512), 0, stream, a);
    else if (a.nsplit > 1 && a.pack)
      hipLaunchKernelGGL((fwd_bf16_kernel<BK, SCORE, 4, 2, 2>), dim3(a.total_wg), dim3(256), 0, stream, a);
    else if (a.nsplit > 1)
      hipLaunchKernelGGL((fwd_bf16_kernel<BK, SCORE, 4, 2, 1>), dim3(a.total_wg), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<BK, SCORE, 4, 2, 0>), dim3(a.total_wg), dim3(256), 0, stream, a);
  } else if (a.total_wg < kF32SplitBelow) {
    // Too few work items to fill the GPU: four workgroups per item, keys split over the waves.
    hipLaunchKernelGGL((fwd_f32_split_kernel<BK, SCORE>), dim3(4 * a.total_wg), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((fwd_f32_kernel<BK, SCORE>), dim3(a.total_wg), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <int BK>
static hipError_t launch_bk(const FwdArgs& a, int dtype, int q_block, int score, hipStream_t stream) {
  switch (score) {
    case 0: return launch_t<BK, 0>(a, dtype, q_block, stream);
    case FA_SCORE_ALIBI: return launch_t<BK, FA_SCORE_ALIBI>(a, dtype, q_block, stream);
    case FA_SCORE_SOFTCAP: return launch_t<BK, FA_SCORE_SOFTCAP>(a, dtype, q_block, stream);
    default: return launch_t<BK, FA_SCORE_ALIBI | FA_SCORE_SOFTCAP>(a, dtype, q_block, stream);
  }
}

// Split-KV merge: one wave per query row; lane l owns channels 2l and 2l + 1. With the ranges'
// lse_s (natural log) and normalised outputs O_s: lse = log sum_s exp(lse_s) and
// O = sum_s exp(lse_s - lse) O_s. A row whose every range is empty keeps O = 0, lse = -inf.
__global__ __launch_bounds__(256) void splitkv_merge_kernel(MergeArgs m) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t nrows = (int64_t)m.B * m.Hq * m.Lq;
  if (row >= nrows) return;
  const int64_t stride = nrows;  // between splits
  float mx = -INFINITY;
  for (int sp = 0; sp < m.nsplit; ++sp) mx = fmaxf(mx, m.part_lse[sp * stride + row]);
  float o0 = 0.f, o1 = 0.f, wsum = 0.f;
  if (mx != -INFINITY) {
    for (int sp = 0; sp < m.nsplit; ++sp) {
      const float ls = m.part_lse[sp * stride + row];
      const float w = ls == -INFINITY ? 0.f : expf(ls - mx);
      const float2 v = *(const float2*)(m.part_o + (sp * stride + row) * 128 + 2 * lane);
      o0 = fmaf(w, v.x, o0);
      o1 = fmaf(w, v.y, o1);
      wsum += w;
    }
    o0 /= wsum;
    o1 /= wsum;
  }
  const int qi = (int)(row % m.Lq);
  const int64_t bh = row / m.Lq;
  const int hq = (int)(bh % m.Hq), b = (int)(bh / m.Hq);
  __bf16* op = m.o + b * m.o_sb + hq * m.o_sh + (int64_t)qi * m.o_sl + 2 * lane;
  op[0] = (__bf16)o0;
  op[1] = (__bf16)o1;
  if (lane == 0 && m.lse) m.lse[row] = mx == -INFINITY ? -INFINITY : mx + logf(wsum);
}

hipError_t launch_splitkv_merge(const MergeArgs& m, hipStream_t stream) {
  const int64_t nrows = (int64_t)m.B * m.Hq * m.Lq;
  if (nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(splitkv_merge_kernel, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, stream, m);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int q_block, int kv_block, int score, hipStream_t stream) {
  if (a.total_wg == 0) return hipSuccess;
  return kv_block == 64 ? launch_bk<64>(a, dtype, q_block, score, stream)
                        : launch_bk<128>(a, dtype, q_block, score, stream);
}

}  // namespace fa

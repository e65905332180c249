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

#include "device_common.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kD = 128;
constexpr int kBQ = 128;

struct WorkItem {
  int b, hq, hkv, qb;
};

__device__ __forceinline__ WorkItem decode_work(const FwdArgs& a) {
  int w = xcd_remap(blockIdx.x, a.total_wg);
  // Order: query heads of one kv head fastest (they read the same K/V tiles), then query
  // blocks from the last (most tiles under causal masks) to the first, then kv head, batch.
  WorkItem it;
  const int g = w % a.group;
  w /= a.group;
  const int qbr = w % a.nqb;
  w /= a.nqb;
  it.hkv = w % a.Hkv;
  it.b = w / a.Hkv;
  it.qb = a.nqb - 1 - qbr;
  it.hq = it.hkv * a.group + g;
  return it;
}

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
// logit. SCORE bits: FA_SCORE_ALIBI, FA_SCORE_SOFTCAP (ALiBi first, then the soft-cap).
template <int SCORE>
__device__ __forceinline__ float score_log2(const FwdArgs& a, float acc, int qi, int kv, float slope) {
  if constexpr (SCORE == 0) {
    return acc * a.scale_log2;
  } else {
    float s = acc * a.sm_scale;
    if constexpr (SCORE & FA_SCORE_ALIBI) s = fmaf(-slope, fabsf((float)(qi - kv)), s);
    if constexpr (SCORE & FA_SCORE_SOFTCAP) s = a.softcap * fast_tanh(s * a.inv_softcap);
    return s * kLog2e;
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------------------------
template <int BK, int SCORE>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int NB = BK / 32;               // 32-key sub-blocks per tile
  constexpr int CHUNKS = BK * 16 / 256;     // 16-byte chunks per thread per K (or V) tile
  __shared__ __attribute__((aligned(16))) unsigned char sK[BK * 256];
  __shared__ __attribute__((aligned(16))) unsigned char sV[BK * 256];
  __shared__ int sDoc[BK];

  const WorkItem it = decode_work(a);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hl = lane >> 5, lq = lane & 31;
  const int qi = it.qb * kBQ + wave * 32 + lq;
  const bool q_in = qi < a.Lq;

  const __bf16* qp = (const __bf16*)a.q + it.b * a.q_sb + it.hq * a.q_sh;
  const __bf16* kp = (const __bf16*)a.k + it.b * a.k_sb + it.hkv * a.k_sh;
  const __bf16* vp = (const __bf16*)a.v + it.b * a.v_sb + it.hkv * a.v_sh;

  // Q^T as the B operand: lane holds Q[qi][16*ks + 8*hl .. +8] for ks = 0..7.
  bf16x8 qreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (q_in) {
      qreg[ks] = *(const bf16x8*)(qp + (int64_t)qi * a.q_sl + ks * 16 + hl * 8);
    } else {
      qreg[ks] = bf16x8{};
    }
  }
  const int qdoc = ((a.flags & FA_MASK_DOC) && q_in) ? a.q_doc[(int64_t)it.b * a.Lq + qi] : 0;
  const float slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[it.hq] : 0.f;
  const MaskSpec ms{a.flags, a.window, a.prefix_len};

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const TileList tl = tile_list(a, it);
  const int ntiles = tl.nfull + tl.npart;

  const int g16 = lane >> 4, s16 = lane & 15;  // 16-lane group and index for transposed reads

  for (int t = 0; t < ntiles; ++t) {
    const bool partial = t >= tl.nfull;
    const int kb = partial ? tl.part[t - tl.nfull] : (a.all_full ? t : tl.full[t]);
    if (kb < 0 || kb >= a.nkvb) continue;  // corrupt index: skip rather than read out of range
    const int kv0 = kb * BK;
    const bool masked = partial || (kv0 + BK > a.Lkv);

    __syncthreads();  // all waves are done reading the previous tile
    {
      bf16x8 kr[CHUNKS], vr[CHUNKS];
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) {
        const int id = tid + c * 256, r = id >> 4, ch = id & 15;
        const int kv = kv0 + r;
        if (kv < a.Lkv) {
          kr[c] = *(const bf16x8*)(kp + (int64_t)kv * a.k_sl + ch * 8);
          vr[c] = *(const bf16x8*)(vp + (int64_t)kv * a.v_sl + ch * 8);
        } else {
          kr[c] = bf16x8{};
          vr[c] = bf16x8{};
        }
      }
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) {
        const int id = tid + c * 256, r = id >> 4, ch = id & 15;
        *(bf16x8*)(sK + tile_off(r, ch)) = kr[c];
        *(bf16x8*)(sV + tile_off(r, ch)) = vr[c];
      }
      if (masked && (a.flags & FA_MASK_DOC) && tid < BK) {
        const int kv = kv0 + tid;
        sDoc[tid] = kv < a.Lkv ? a.kv_doc[(int64_t)it.b * a.Lkv + kv] : 0;
      }
    }
    __syncthreads();

    // S^T = K Q^T for NB sub-blocks of 32 keys.
    f32x16 sacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      sacc[nb] = f32x16{};
      const int r = nb * 32 + lq;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(sK + tile_off(r, 2 * ks + hl));
        sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[ks], sacc[nb], 0, 0, 0);
      }
    }

    // Scores in the log2 domain, mask on partial (and ragged) tiles, running max.
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

    // P = exp2(t - m); P^T goes straight into the B operand of O^T = V^T P^T as bf16.
    float rs = 0.f;
    bf16x8 pb[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(sacc[nb][i] - m_use);
        rs += p;
        pb[nb][i >> 3][i & 7] = (__bf16)p;
      }
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T. A operand (V^T, row = channel d, k = key) via transposed LDS reads: in each
    // 16-lane group, source lane s points at row (key) base + s/4, channels d0 + 4*(s%4); lane i
    // of the group then receives V[base + j][d0 + i] for j = 0..3.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + 16 * (g16 & 1) + 4 * (s16 & 3);
      const int ch = d >> 3, boff = (d & 7) * 2;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r0 = nb * 32 + h * 16 + (g16 >> 1) * 4 + (s16 >> 2);
          const int r1 = r0 + 8;
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(sV + tile_off(r0, ch) + boff));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(sV + tile_off(r1, ch) + boff));
          // Whole-vector concatenation and bit cast (element-wise bf16 inserts of the i16
          // lanes were observed to be folded into a broadcast of element 0).
          const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, cat);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[nb][h], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // Epilogue: combine the two halves' row sums, normalise, store O (bf16) and the natural-log lse.
  const float l_tot = half_swap_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_in) {
    __bf16* op = (__bf16*)a.o + it.b * a.o_sb + it.hq * a.o_sh + (int64_t)qi * a.o_sl;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 o4;
        o4[0] = (__bf16)(oacc[db][gq * 4 + 0] * inv);
        o4[1] = (__bf16)(oacc[db][gq * 4 + 1] * inv);
        o4[2] = (__bf16)(oacc[db][gq * 4 + 2] * inv);
        o4[3] = (__bf16)(oacc[db][gq * 4 + 3] * inv);
        *(bf16x4*)(op + db * 32 + gq * 8 + hl * 4) = o4;
      }
    }
    if (a.lse && hl == 0) {
      a.lse[((int64_t)it.b * a.Hq + it.hq) * a.Lq + qi] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
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

  const WorkItem it = decode_work(a);
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
  const float slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[it.hq] : 0.f;
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
    for (int id = tid; id < BK * 32; id += 256) {  // float4 chunks
      const int r = id >> 5, c4 = id & 31;
      const int kv = kv0 + r;
      f32x4 kx = f32x4{}, vx = f32x4{};
      if (kv < a.Lkv) {
        kx = *(const f32x4*)(kp + (int64_t)kv * a.k_sl + c4 * 4);
        vx = *(const f32x4*)(vp + (int64_t)kv * a.v_sl + c4 * 4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sK[r * P + c4 * 4 + e] = kx[e];
        sV[r * P + c4 * 4 + e] = vx[e];
      }
    }
    if (masked && (a.flags & FA_MASK_DOC) && tid < BK) {
      const int kv = kv0 + tid;
      sDoc[tid] = kv < a.Lkv ? a.kv_doc[(int64_t)it.b * a.Lkv + kv] : 0;
    }
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

// ---------------------------------------------------------------------------------------------
template <int BK, int SCORE>
static hipError_t launch_t(const FwdArgs& a, int dtype, hipStream_t stream) {
  if (dtype == 1) {
    hipLaunchKernelGGL((fwd_bf16_kernel<BK, SCORE>), dim3(a.total_wg), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((fwd_f32_kernel<BK, SCORE>), dim3(a.total_wg), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <int BK>
static hipError_t launch_bk(const FwdArgs& a, int dtype, int score, hipStream_t stream) {
  switch (score) {
    case 0: return launch_t<BK, 0>(a, dtype, stream);
    case FA_SCORE_ALIBI: return launch_t<BK, FA_SCORE_ALIBI>(a, dtype, stream);
    case FA_SCORE_SOFTCAP: return launch_t<BK, FA_SCORE_SOFTCAP>(a, dtype, stream);
    default: return launch_t<BK, FA_SCORE_ALIBI | FA_SCORE_SOFTCAP>(a, dtype, stream);
  }
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int kv_block, int score, hipStream_t stream) {
  if (a.total_wg == 0) return hipSuccess;
  return kv_block == 64 ? launch_bk<64>(a, dtype, score, stream) : launch_bk<128>(a, dtype, score, stream);
}

}  // namespace fa

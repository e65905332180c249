// Block-sparse masked attention backward for gfx950 (CDNA4), bf16, head dim 128.
//
// Method (FlexAttention guide, "Systems Mechanics", item 2): the backward of the fused forward
// gives dQ, dK and dV, differentiates the score_mod, and lets gradients reach learnable score_mod
// parameters (ALiBi slopes). It walks the same BlockMask tiles as the forward: full tiles without
// the mask, partial tiles with it, empty tiles never.
//
// With r = q.k (raw product), s = r * sm_scale, a = s - slope |i - j| (ALiBi), f = C tanh(a / C)
// (soft-cap, else f = a), P = exp(f - lse) on allowed pairs and 0 elsewhere:
//   dV = P^T dO,  dP = dO V^T,  dF = P (dP - delta), delta_i = dO_i . O_i,
//   dA = dF (1 - (f / C)^2)  (soft-cap; dA = dF without),  dslope_h = -sum dA |i - j|,
//   dQ = sm_scale dA K,  dK = sm_scale dA^T Q.
// P is recomputed from the forward's lse, so nothing of size Lq x Lkv is stored.
//
// Kernels:
//   bwd_dq_kernel       one workgroup of 4 waves per (b, query head, 128-query block), walking the
//                       row's BlockMask tiles in steps of 64 keys. Orientation of the forward:
//                       each wave computes S^T = K Q^T and dP^T = V dO^T with Q^T and dO^T held
//                       in registers as B operands (a lane owns one query), then
//                       dQ^T += K^T dA^T with dA^T straight from the accumulators as the B
//                       operand and K^T read from LDS with ds_read_b64_tr_b16. K and V tiles
//                       stream into two LDS buffers by global_load_lds, one step ahead; two
//                       waves per SIMD. Its prologue computes each row's delta = dO . O and
//                       lse2 = lse * log2(e) (+inf for a row with no allowed key, so its
//                       probabilities are exactly 0) and writes them for the dK/dV pass, which
//                       runs after it. Also sums the ALiBi-slope gradient of its rows;
//   bwd_dkdv_kernel     one workgroup of 4 waves per (b, kv head, 128-key block), walking the
//                       column's q blocks (the transposed BlockMask) for every query head of the
//                       group, in steps of 64 queries. Mirrored orientation: S = Q K^T and
//                       dP = dO V^T with K^T and V^T held in registers (a lane owns one key),
//                       then dV^T += dO^T P and dK^T += Q^T dA, both A operands read transposed
//                       from LDS. GQA sums over the group inside the workgroup (no atomics).
//                       K^T, V^T and both accumulators hold 192 registers, so it runs at one
//                       wave per SIMD; Q and dO tiles of a whole 128-query block per step are
//                       staged through registers (with LDS-DMA at one wave per SIMD, issuing the
//                       transfers stalled the only wave and measured slower; splitting dK and dV
//                       into two kernels spilled);
//   bwd_slope_kernel    sums the per-block slope partials into dslopes[h] (deterministic).
//
// Accumulator layout (32x32 MFMA): element i of lane l holds row 8*(i/4) + 4*(l/32) + i%4 and
// column l%32. Tiles in LDS are [rows][128 bf16] with 16-byte chunks XOR-swizzled by row
// (tile_off), which serves both the row reads of A operands and the transposed reads.
#include <hip/hip_runtime.h>

#include <climits>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kRows = 64;                  // rows per LDS tile and per step

// Position w of the (batch, kv head) pairs in dispatch order -> pair index: the XCDs receive
// contiguous ranges of work, and range c holds pairs c, c + 8, c + 16, ..., so every XCD mixes
// batches (whose document structures, and work, differ).
__device__ __forceinline__ int permute_pair(int w, int npair) {
  const int q8 = npair / 8, r8 = npair % 8;
  int c, k;
  if (w < r8 * (q8 + 1)) {
    c = w / (q8 + 1);
    k = w % (q8 + 1);
  } else {
    c = r8 + (w - r8 * (q8 + 1)) / q8;
    k = (w - r8 * (q8 + 1)) % q8;
  }
  return 8 * k + c;
}
constexpr int kTileBytes = kRows * 256;    // [64][128] bf16
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Transposed-read base offset of this lane (see the forward kernel): in each 16-lane group,
// source lane s points at row (g/2)*4 + s/4 and channels 16*(g%2) + 4*(s%4); lane i of the
// group then receives X[row0 + j][d0 + i], j = 0..3.
__device__ __forceinline__ int tr_base(int lane) {
  const int g16 = lane >> 4, s16 = lane & 15;
  const int d = 16 * (g16 & 1) + 4 * (s16 & 3);
  const int r0 = (g16 >> 1) * 4 + (s16 >> 2);
  return tile_off(r0, d >> 3) + (d & 7) * 2;
}

// Operand offsets. The swizzle's fields are disjoint bit ranges of the byte offset, so every
// operand read of a step is one per-lane base XORed with a constant: row reads (A operand X,
// row lq, channels 16 ks + 8 hl) at kx0 ^ 32 ks; transposed reads of channel block db and
// rows + 8 j at tb ^ (64 db + 2080 j). Row blocks of 16 add multiples of 4096 bytes (the
// swizzle depends on the row modulo 16 only), which fold into the instruction's offset. The
// bases are re-defined per step by an empty asm, so the compiler keeps one register each
// instead of one per (buffer, offset) pair.
__device__ __forceinline__ int launder(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A operand of X^T (row = channel in block db, k = 16 tile rows from row0, in the order of the
// accumulator rows i = 8h .. 8h+7 of a 32x32 tile) from a swizzled [rows][128] tile.
__device__ __forceinline__ bf16x8 read_xt(const unsigned char* tile, int row0, int db, int tb) {
  const unsigned char* base = tile + row0 * 256;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + (tb ^ (64 * db))));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + (tb ^ (64 * db + 2080))));
  const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, cat);
}

// A operand of X (row = row0 + lq, k = channels 16 ks + 8 hl .. +8); kx0 = tile_off(lq, hl).
__device__ __forceinline__ bf16x8 read_x(const unsigned char* tile, int row0, int ks, int kx0) {
  return *(const bf16x8*)(tile + row0 * 256 + (kx0 ^ (32 * ks)));
}

template <class F, int... I>
__device__ __forceinline__ void bwd_static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, class F>
__device__ __forceinline__ void bwd_static_for(F&& f) {
  bwd_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Score and its derivative factor for one pair: returns f (natural units) and sets dfac =
// d f / d a (1 - tanh^2 under soft-cap, else 1).
template <int SCORE>
__device__ __forceinline__ float score_f(const BwdArgs& a, float r, int qi, int kv, float slope, float& dfac) {
  float s = r * a.sm_scale;
  if constexpr (SCORE & FA_SCORE_ALIBI) s = fmaf(-slope, fabsf((float)(qi - kv)), s);
  dfac = 1.0f;
  if constexpr (SCORE & FA_SCORE_SOFTCAP) {
    const float th = fast_tanh(s * a.inv_softcap);
    dfac = 1.0f - th * th;
    s = a.softcap * th;
  }
  return s;
}

// Branch-free mask_mod for one pair (the predicates of the forward, evaluated with selects so
// that partial tiles compile to straight-line code). With d = i - j: CAUSAL needs d >= 0,
// WINDOW d <= window - 1, PREFIX_LM d >= 0 unless j < prefix_len, DOC equal ids.
struct PairMask {
  int dlo, dhi, prefix_len;
  bool prefix, doc;
};

__device__ __forceinline__ PairMask make_pair_mask(const BwdArgs& a) {
  PairMask m;
  m.dlo = (a.flags & FA_MASK_CAUSAL) ? 0 : INT_MIN;
  m.dhi = (a.flags & FA_MASK_WINDOW) ? a.window - 1 : INT_MAX;
  m.prefix = (a.flags & FA_MASK_PREFIX_LM) != 0;
  m.prefix_len = a.prefix_len;
  m.doc = (a.flags & FA_MASK_DOC) != 0;
  return m;
}

__device__ __forceinline__ bool pair_ok(const PairMask& m, int i, int j, int qd, int kd) {
  const int d = i - j;
  const int lo = (m.prefix & (j >= m.prefix_len)) ? 0 : m.dlo;
  return (d >= lo) & (d <= m.dhi) & (!m.doc | (qd == kd));
}

// Schedules of the product chains (scheduling-group masks: 0x008 MFMA, 0x100 LDS read): the
// operand reads run at most a few products ahead instead of all at once, which would hold up to
// 64 registers of operands in flight.
// N pairs of products with one 16-byte read each: 4 reads ahead, then 2 products per 2 reads.
template <int N> __device__ __forceinline__ void sched_pairs() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (k + 2 < N) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}
// N products with two transposed 8-byte reads each: 2 products' reads ahead, then 1 product
// per 2 reads.
template <int N> __device__ __forceinline__ void sched_tr() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (k + 2 < N) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// Stage rows [r0, r0 + ROWS) of two [L][128] bf16 tensors into registers (ROWS / 16 chunks of
// 16 bytes per thread and tensor); rows at or past L read row L - 1 and are zeroed when stored.
template <int ROWS>
struct Stage {
  static constexpr int U = ROWS * 16 / 256;
  i32x4 x[U], y[U];
};

template <int ROWS>
__device__ __forceinline__ void stage_load(Stage<ROWS>& st, const __bf16* xp, int64_t xsl, const __bf16* yp,
                                           int64_t ysl, int r0, int L, int tid) {
#pragma unroll
  for (int u = 0; u < Stage<ROWS>::U; ++u) {
    const int id = tid + 256 * u;
    const int r = min(r0 + (id >> 4), L - 1);
    const int ch = id & 15;
    st.x[u] = *(const i32x4*)(xp + (int64_t)r * xsl + ch * 8);
    st.y[u] = *(const i32x4*)(yp + (int64_t)r * ysl + ch * 8);
  }
}

template <int ROWS>
__device__ __forceinline__ void stage_store(const Stage<ROWS>& st, unsigned char* sx, unsigned char* sy, int r0, int L,
                                            int tid) {
#pragma unroll
  for (int u = 0; u < Stage<ROWS>::U; ++u) {
    const int id = tid + 256 * u;
    const int r = id >> 4, ch = id & 15;
    const bool in = r0 + r < L;
    *(i32x4*)(sx + tile_off(r, ch)) = in ? st.x[u] : i32x4{0, 0, 0, 0};
    *(i32x4*)(sy + tile_off(r, ch)) = in ? st.y[u] : i32x4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Tile transfers. Each step moves 64 rows of two [L][128] bf16 tensors into LDS with
// global_load_lds_dwordx4 (LDS written directly, no registers): 16 one-KB segments of 4 rows per
// tensor, segment 4 i + wave issued by that wave. Lane l of a segment writes LDS chunk slot
// l % 16 of row l / 16; it loads global chunk slot ^ swz(row), so the tile lands swizzled. Rows
// at or past the end re-read the last row (finite data; the kernels mask them). Row-wise values
// (16 per wave) follow as 4-byte transfers; every step issues the same number of transfers per
// wave, so waiting for a step is one s_waitcnt vmcnt with a constant count.
// ---------------------------------------------------------------------------------------------
namespace {

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}
// The compiler does not track the LDS writes of global_load_lds: at most N vector-memory
// operations of this wave may still be outstanding after this. Emitted with the builtin, whose
// encoding the compiler reads (vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at
// their maxima), so that it also knows the older transfers are complete; an asm wait is opaque
// to it, and it then waited for every transfer before reading a buffer filled earlier.
template <int N> __device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier without the memory fence of __syncthreads(): that fence makes the compiler
// wait for every outstanding transfer into LDS (vmcnt(0)), including the next step's, which then
// never overlaps the current step. Each wave waits for its own transfers of the step explicitly
// (wait_vmem), and its LDS reads of a step have returned before their products or vector work;
// the empty asm statements keep the compiler from moving LDS accesses or transfers across.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Lane {
  int wave, lane, hl, lq;
  int r_l;   // row of this lane in its first segment (4 wave + lane / 16); later segments add 16
  int ch;    // global chunk this lane loads (slot ^ swz(row), the same for every segment)
  int tb;    // transposed-read base offset
  int kx0;   // row-read base offset, tile_off(lq, hl)
};

__device__ __forceinline__ Lane make_lane() {
  Lane c;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.hl = c.lane >> 5;
  c.lq = c.lane & 31;
  c.r_l = 4 * c.wave + (c.lane >> 4);
  c.ch = (c.lane & 15) ^ swz(c.r_l);
  c.tb = tr_base(c.lane);
  c.kx0 = tile_off(c.lq, c.hl);
  return c;
}

// 8 transfers: rows [r0, r0 + 64) of x and y (row strides xsl, ysl). xoff / yoff are the lane's
// element offsets in its first segment (r_l * stride + ch * 8), so the address of a full step is
// a uniform base plus one 32-bit lane offset; a step reaching past row L - 1 clamps per row.
__device__ __forceinline__ void issue_tiles(const Lane& c, const __bf16* xp, int64_t xsl, int xoff, const __bf16* yp,
                                            int64_t ysl, int yoff, int r0, int L, unsigned char* sx,
                                            unsigned char* sy) {
  if (r0 + kRows <= L) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int seg = 4 * i + c.wave;
      dma16(xp + (int64_t)(r0 + 16 * i) * xsl + xoff, sx + seg * 1024);
      dma16(yp + (int64_t)(r0 + 16 * i) * ysl + yoff, sy + seg * 1024);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = min(r0 + c.r_l + 16 * i, L - 1);
      const int seg = 4 * i + c.wave;
      dma16(xp + r * xsl + c.ch * 8, sx + seg * 1024);
      dma16(yp + r * ysl + c.ch * 8, sy + seg * 1024);
    }
  }
}

// 1 transfer: 16 row-wise 4-byte values per wave (rows r0 + 16 wave + lane, clamped), from
// base[row]; base may be a valid dummy address when the values are unused.
__device__ __forceinline__ void issue_rowvals(const Lane& c, const void* base, bool use, int r0, int L, void* dst) {
  if (c.lane < 16) {
    const char* src = (const char*)base + (use ? 4 * (int64_t)min(r0 + 16 * c.wave + c.lane, L - 1) : 0);
    dma4(src, (char*)dst + 64 * c.wave);
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// dQ (and the slope-gradient partials): one workgroup per (b, hq, 128-query block).
// ---------------------------------------------------------------------------------------------

template <int SCORE>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char sK0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sV0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sK1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sV1[kTileBytes];
  __shared__ __attribute__((aligned(16))) int sD0[kRows];
  __shared__ __attribute__((aligned(16))) int sD1[kRows];
  __shared__ float sRed[4];
  constexpr int kOps = 9;  // transfers per wave and step

  // Order: query heads of one kv head fastest (they read the same K/V tiles), then query blocks
  // from last to first (the longest rows under causal masks first), then (batch, kv head)
  // pairs; each XCD takes one contiguous range, the pairs permuted so that ranges mix batches.
  // With the BlockMask's schedule: rank r of the row order outermost (the costliest query
  // blocks first), then (batch, kv head) pairs, then the query heads of a kv head, dealt
  // round-robin to the XCDs as the forward does.
  int qb, hq, hkv, b;
  if (a.row_order != nullptr) {
    const int npair = a.B * a.Hkv, per_rank = npair * a.group;
    const int idx = blockIdx.x % per_rank, r = blockIdx.x / per_rank;
    const int pair = idx % npair, g = idx / npair;
    hkv = pair % a.Hkv;
    b = pair / a.Hkv;
    hq = hkv * a.group + g;
    qb = min(max(a.row_order[(int64_t)(a.Bm == 1 ? 0 : b) * a.nqb + r], 0), a.nqb - 1);
  } else {
    int w = xcd_remap(blockIdx.x, (int)((int64_t)a.B * a.Hq * a.nqb));
    const int g = w % a.group;
    w /= a.group;
    qb = a.nqb - 1 - (w % a.nqb);
    w /= a.nqb;
    const int pair = permute_pair(w, a.B * a.Hkv);
    hkv = pair % a.Hkv;
    b = pair / a.Hkv;
    hq = hkv * a.group + g;
  }
  // Wave-uniform, but computed by vector divisions: in scalar registers the K, V and document
  // pointers derived from them stay scalar too (in vector registers they were spilled, and each
  // reload inside a step's transfers waited for all of them).
  qb = __builtin_amdgcn_readfirstlane(qb);
  hq = __builtin_amdgcn_readfirstlane(hq);
  hkv = __builtin_amdgcn_readfirstlane(hkv);
  b = __builtin_amdgcn_readfirstlane(b);
  const Lane c = make_lane();
  const int hl = c.hl, lq = c.lq;
  const int qi = qb * 128 + c.wave * 32 + lq;
  const bool q_in = qi < a.Lq;
  const int qc = min(qi, a.Lq - 1);
  const bool doc = (a.flags & FA_MASK_DOC) != 0;

  // Q^T and dO^T as B operands: lane holds X[qi][16 ks + 8 hl .. +8].
  const __bf16* qp = (const __bf16*)a.q + b * a.q_sb + hq * a.q_sh + (int64_t)qc * a.q_sl;
  const __bf16* dop = (const __bf16*)a.dout + b * a.do_sb + hq * a.do_sh + (int64_t)qc * a.do_sl;
  bf16x8 qreg[8], doreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qreg[ks] = *(const bf16x8*)(qp + ks * 16 + hl * 8);
    doreg[ks] = *(const bf16x8*)(dop + ks * 16 + hl * 8);
  }
  const int64_t row = ((int64_t)b * a.Hq + hq) * a.Lq + qc;
  // delta = dO . O of the row (the lane's 64 channels, then the other half's by lane swap) and
  // lse2 = lse * log2(e), +inf for a row with no allowed key. Written for the dK/dV pass.
  float lse2, delta;
  {
    const __bf16* orow = (const __bf16*)a.o + b * a.o_sb + hq * a.o_sh + (int64_t)qc * a.o_sl;
    float dacc = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 o8 = *(const bf16x8*)(orow + ks * 16 + hl * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) dacc = fmaf((float)o8[e], (float)doreg[ks][e], dacc);
    }
    const float dfull = half_swap_sum(dacc);
    const float l = a.lse[row];
    lse2 = q_in ? (l == -INFINITY ? INFINITY : l * kLog2e) : INFINITY;
    delta = q_in ? dfull : 0.f;
    if (q_in && hl == 0) {
      a.delta[row] = delta;
      a.lse2[row] = lse2;
    }
  }
  const int qdoc = doc ? a.q_doc[(int64_t)b * a.Lq + qc] : 0;
  const float slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[hq] : 0.f;
  const PairMask pm = make_pair_mask(a);

  const __bf16* kp = (const __bf16*)a.k + b * a.k_sb + hkv * a.k_sh;
  const __bf16* vp = (const __bf16*)a.v + b * a.v_sb + hkv * a.v_sh;
  const int* kvdoc = doc ? a.kv_doc + (int64_t)b * a.Lkv : (const int*)kp;
  const int koff = c.r_l * (int)a.k_sl + c.ch * 8, voff = c.r_l * (int)a.v_sl + c.ch * 8;

  int nfull, npart;
  const int* full = nullptr;
  const int* part = nullptr;
  if (a.all_full) {
    nfull = (a.Lkv + 127) / 128;
    npart = 0;
  } else {
    const int bm = a.Bm == 1 ? 0 : b;
    const int64_t r = (int64_t)bm * a.nqb + qb;
    nfull = clamp_count(a.full_num[r], a.nkvb);
    npart = clamp_count(a.kv_num[r], a.nkvb);
    full = a.full_idx + r * a.nkvb;
    part = a.kv_idx + r * a.nkvb;
  }
  const int nsteps = 2 * (nfull + npart);
  // List entries, 64 per register: lane j holds the key block of tile chunk_base + j (without a
  // BlockMask, block t itself). Steps are looked up in increasing order (each once, when it is
  // issued), so the register moves forward only.
  const int ntiles = nfull + npart;
  auto load_chunk = [&](int base) -> int {
    const int t = base + c.lane;
    if (a.all_full || t >= ntiles) return t;
    return t < nfull ? full[t] : part[t - nfull];
  };
  int chunk_base = 0;
  int chunk = load_chunk(0);
  auto step_kv0 = [&](int s, bool& masked) {
    const int t = s >> 1;
    if (t >= chunk_base + 64) {
      chunk_base = t & ~63;
      chunk = load_chunk(chunk_base);
      asm volatile("" ::"v"(chunk));  // waited for here, not at every step's readlane
    }
    const bool partial = t >= nfull;
    // An entry outside [0, n_kvb) becomes n_kvb: its rows lie past the keys, so the transfers
    // clamp to the last key and every score of the step is masked (it adds nothing).
    const int kb = a.all_full ? t : sanitize_block(__builtin_amdgcn_readlane(chunk, t - chunk_base), a.nkvb);
    const int kv0 = kb * 128 + (s & 1) * kRows;
    masked = partial || kv0 + kRows > a.Lkv;
    return kv0;
  };
  auto issue = [&](int kv0, unsigned char* sK, unsigned char* sV, int* sD) {
    // Everything the transfers need is materialised before the first of them: the uniform bases
    // in scalar registers and the lane offsets re-defined here (hoisted, pointer plus offset
    // became one 64-bit register per tensor, kept across the loop and spilled). A value reloaded
    // from scratch between two transfers waits for both, which leaves nothing in flight.
    const __bf16* kpu = kp;
    const __bf16* vpu = vp;
    const int* kdu = kvdoc;
    asm volatile("" : "+s"(kpu), "+s"(vpu), "+s"(kdu));
    const int ko = launder(koff), vo = launder(voff);
    issue_rowvals(c, kdu, doc, kv0, a.Lkv, sD);
    issue_tiles(c, kpu, a.k_sl, ko, vpu, a.v_sl, vo, kv0, a.Lkv, sK, sV);
  };

  f32x16 dqacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dqacc[db] = f32x16{};
  float slope_acc = 0.f;

  auto compute = [&](int kv0, bool masked, const unsigned char* sK, const unsigned char* sV, const int* sD) {
    // The V reads take their own copy of the offset: with one, the compiler formed the V address
    // as the K address plus the distance between the arrays, lost track of which buffer it reads,
    // and waited for every transfer in flight (the next step's) before it.
    const int kx0 = launder(c.kx0), kxv = launder(c.kx0), tb = launder(c.tb);
#pragma unroll 1
    for (int nb = 0; nb < 2; ++nb) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_x(sK, nb * 32, ks, kx0), qreg[ks], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_x(sV, nb * 32, ks, kxv), doreg[ks], dpacc, 0, 0, 0);
      }
      sched_pairs<8>();
      bf16x8 dsb[2];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int kr4 = nb * 32 + 8 * gq + 4 * hl;
        const i32x4 d4 = *(const i32x4*)(sD + kr4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * gq + e;
          const int kv = kv0 + kr4 + e;
          float dfac;
          const float f = score_f<SCORE>(a, sacc[i], qi, kv, slope, dfac);
          float p = fast_exp2(fmaf(f, kLog2e, -lse2));
          if (masked) p = ((kv < a.Lkv) & pair_ok(pm, qi, kv, qdoc, d4[e])) ? p : 0.f;
          float da = p * (dpacc[i] - delta);
          if constexpr (SCORE & FA_SCORE_SOFTCAP) da *= dfac;
          if constexpr (SCORE & FA_SCORE_ALIBI) slope_acc = fmaf(-da, fabsf((float)(qi - kv)), slope_acc);
          dsb[i >> 3][i & 7] = (__bf16)da;
        }
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_xt(sK, nb * 32 + h * 16, db, tb), dsb[h],
                                                              dqacc[db], 0, 0, 0);
      }
      sched_tr<8>();
    }
  };

  // Two LDS buffers, selected at compile time (the loop handles two steps per iteration):
  // step s + 1 is issued into the other buffer before step s is waited for and computed.
  // The row's operands are complete before the first transfer: loads still pending at the loop
  // made the compiler wait for every outstanding transfer (vmcnt(0)) at their first use in each
  // step, the next step's included.
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qreg[ks]), "v"(doreg[ks]));
  asm volatile("" ::"v"(lse2), "v"(delta), "v"(qdoc), "v"(chunk));
  // Each step's key offset is looked up once, when it is issued, and kept for its compute.
  bool m0 = false, m1 = false;
  int kv_0 = 0, kv_1 = 0;
  if (nsteps > 0) {
    kv_0 = step_kv0(0, m0);
    issue(kv_0, sK0, sV0, sD0);
  }
  for (int s = 0; s < nsteps; s += 2) {
    if (s + 1 < nsteps) {
      kv_1 = step_kv0(s + 1, m1);
      issue(kv_1, sK1, sV1, sD1);
      wait_vmem<kOps>();
    } else {
      wait_vmem<0>();
    }
    step_barrier();
    compute(kv_0, m0, sK0, sV0, sD0);
    step_barrier();
    if (s + 1 >= nsteps) break;
    if (s + 2 < nsteps) {
      kv_0 = step_kv0(s + 2, m0);
      issue(kv_0, sK0, sV0, sD0);
      wait_vmem<kOps>();
    } else {
      wait_vmem<0>();
    }
    step_barrier();
    compute(kv_1, m1, sK1, sV1, sD1);
    step_barrier();
  }
  wait_vmem<0>();  // no transfer may outlive the workgroup's LDS

  // dQ[qi][channel]: lane holds channels 32 db + 8 gq + 4 hl + 0..3 of its query. The rows go out
  // through LDS so that each store writes whole 256-byte rows (from the registers, each store
  // wrote 16 bytes into each of 32 rows): waves 0-1 stage their 32 rows in the first K tile,
  // waves 2-3 in the first V tile (every wave has passed the barrier after its last step), and
  // each wave reads back only its own rows.
  {
    unsigned char* const ob = (c.wave < 2 ? sK0 : sV0) + (c.wave & 1) * (32 * 256);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(dqacc[db][gq * 4 + e] * a.sm_scale);
        *(bf16x4*)(ob + tile_off(lq, db * 4 + gq) + hl * 8) = o4;
      }
    }
    __bf16* const op0 = (__bf16*)a.dq + b * a.dq_sb + hq * a.dq_sh;
    const int qw0 = qb * 128 + c.wave * 32;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (c.lane >> 4), ch = c.lane & 15;
      const bf16x8 v8 = *(const bf16x8*)(ob + tile_off(r, ch));
      if (qw0 + r < a.Lq) *(bf16x8*)(op0 + (int64_t)(qw0 + r) * a.dq_sl + ch * 8) = v8;
    }
  }
  if constexpr (SCORE & FA_SCORE_ALIBI) {
    if (a.dslopes) {
      const float ws = wave_sum(slope_acc);
      if (c.lane == 0) sRed[c.wave] = ws;
      __syncthreads();
      if (threadIdx.x == 0) a.slope_part[((int64_t)b * a.Hq + hq) * a.nqb + qb] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dK and dV: one workgroup per (b, hkv, 128-key block), summing over the query heads of the
// group.
// ---------------------------------------------------------------------------------------------
template <int SCORE>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  // One step takes a whole 128-query block (two 64-row halves took one exposed round trip of
  // staging loads each, at one wave per SIMD).
  constexpr int QR = 128;
  __shared__ __attribute__((aligned(1024))) unsigned char sQ[QR * 256];
  __shared__ __attribute__((aligned(1024))) unsigned char sO[QR * 256];
  __shared__ __attribute__((aligned(16))) float sL[QR];
  __shared__ __attribute__((aligned(16))) float sDl[QR];
  __shared__ __attribute__((aligned(16))) int sDoc[QR];

  // Order: key blocks from first to last (the longest columns under causal masks first), then
  // (batch, kv head) pairs; each XCD takes one contiguous range, pairs permuted as in dQ.
  // With the transposed BlockMask's column schedule: rank r outermost (the costliest columns
  // first), (batch, kv head) pairs fastest, dealt round-robin to the XCDs.
  int kb, hkv, b;
  if (a.col_order != nullptr) {
    const int npair = a.B * a.Hkv;
    const int pair = blockIdx.x % npair, r = blockIdx.x / npair;
    hkv = pair % a.Hkv;
    b = pair / a.Hkv;
    kb = min(max(a.col_order[(int64_t)(a.Bm == 1 ? 0 : b) * a.nkvb + r], 0), a.nkvb - 1);
  } else {
    int w = xcd_remap(blockIdx.x, (int)((int64_t)a.B * a.Hkv * a.nkvb));
    kb = w % a.nkvb;
    w /= a.nkvb;
    const int pair = permute_pair(w, a.B * a.Hkv);
    hkv = pair % a.Hkv;
    b = pair / a.Hkv;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, lq = lane & 31;
  const int kj = kb * 128 + wave * 32 + lq;
  const bool k_in = kj < a.Lkv;
  const int kc = min(kj, a.Lkv - 1);
  const bool doc = (a.flags & FA_MASK_DOC) != 0;

  // K^T and V^T as B operands: lane holds X[kj][16 ks + 8 hl .. +8].
  const __bf16* kp = (const __bf16*)a.k + b * a.k_sb + hkv * a.k_sh + (int64_t)kc * a.k_sl;
  const __bf16* vp = (const __bf16*)a.v + b * a.v_sb + hkv * a.v_sh + (int64_t)kc * a.v_sl;
  bf16x8 kreg[8], vreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kreg[ks] = *(const bf16x8*)(kp + ks * 16 + hl * 8);
    vreg[ks] = *(const bf16x8*)(vp + ks * 16 + hl * 8);
  }
  const int kdoc = doc ? a.kv_doc[(int64_t)b * a.Lkv + kc] : 0;
  const PairMask pm = make_pair_mask(a);
  const int tb = tr_base(lane), kx0 = tile_off(lq, hl);

  f32x16 dkacc[4], dvacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  for (int g = 0; g < a.group; ++g) {
    const int hq = hkv * a.group + g;
    const float slope = (SCORE & FA_SCORE_ALIBI) ? a.slopes[hq] : 0.f;
    const __bf16* qp = (const __bf16*)a.q + b * a.q_sb + hq * a.q_sh;
    const __bf16* dop = (const __bf16*)a.dout + b * a.do_sb + hq * a.do_sh;
    const int64_t rowbase = ((int64_t)b * a.Hq + hq) * a.Lq;

    int nfull, npart;
    const int* full = nullptr;
    const int* part = nullptr;
    if (a.all_full) {
      nfull = (a.Lq + 127) / 128;
      npart = 0;
    } else {
      const int bm = a.Bm == 1 ? 0 : b, hm = a.Hm == 1 ? 0 : hq;
      const int64_t r = ((int64_t)bm * a.Hm + hm) * a.nkvb + kb;
      nfull = clamp_count(a.fullq_num[r], a.nqb);
      npart = clamp_count(a.q_num[r], a.nqb);
      full = a.fullq_idx + r * a.nqb;
      part = a.q_idx + r * a.nqb;
    }
    const int nsteps = nfull + npart;
    for (int t = 0; t < nsteps; ++t) {
      const bool masked = t >= nfull;
      // An entry outside [0, n_qb) becomes n_qb, whose rows lie past the queries: skipped.
      const int qbk = masked ? sanitize_block(part[t - nfull], a.nqb) : (a.all_full ? t : sanitize_block(full[t], a.nqb));
      const int q0 = qbk * 128;
      if (q0 >= a.Lq) continue;  // uniform over the workgroup

      Stage<QR> st;
      stage_load<QR>(st, qp, a.q_sl, dop, a.do_sl, q0, a.Lq, tid);
      float lv = INFINITY, dv = 0.f;
      int dd = 0;
      if (tid < QR) {
        const int qr = q0 + tid;
        if (qr < a.Lq) {
          lv = a.lse2[rowbase + qr];
          dv = a.delta[rowbase + qr];
          if (doc) dd = a.q_doc[(int64_t)b * a.Lq + qr];
        }
      }
      __syncthreads();  // the previous step's reads are done
      stage_store<QR>(st, sQ, sO, q0, a.Lq, tid);
      if (tid < QR) {
        sL[tid] = lv;
        sDl[tid] = dv;
        sDoc[tid] = dd;
      }
      __syncthreads();

      // The step's four 32-query sub-blocks, software-pipelined: while sub-block s's vector work
      // turns its scores into P and dA, the MFMA pipe runs the dV/dK products of sub-block s - 1
      // and the S^T/dP^T products of sub-block s + 1. The order is fixed at compile time: each
      // slot (one score's vector work and one pair of products) ends with a scheduling barrier.
      // Full and partial tiles share this code; a partial tile's P and dA are masked afterwards
      // (a select per score), before its dV/dK products.
      f32x16 sa[2], da[2];        // S^T and dP^T of sub-blocks s (s % 2)
      bf16x8 pb[2][2], dsb[2][2];  // P and dA of sub-blocks s (s % 2), as B operands
      auto sdp = [&](auto sc, auto kc) {  // S^T / dP^T products of k-step ks
        constexpr int sb = decltype(sc)::value, ks = decltype(kc)::value;
        sa[sb & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_x(sQ, sb * 32, ks, kx0), kreg[ks],
                                                             ks ? sa[sb & 1] : f32x16{}, 0, 0, 0);
        da[sb & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_x(sO, sb * 32, ks, kx0), vreg[ks],
                                                             ks ? da[sb & 1] : f32x16{}, 0, 0, 0);
      };
      auto dkv = [&](auto sc, auto jc) {  // dV / dK products of channel block j / 2, key half j % 2
        constexpr int sb = decltype(sc)::value, j = decltype(jc)::value;
        constexpr int db = j >> 1, h = j & 1;
        dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_xt(sO, sb * 32 + h * 16, db, tb), pb[sb & 1][h],
                                                            dvacc[db], 0, 0, 0);
        dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_xt(sQ, sb * 32 + h * 16, db, tb), dsb[sb & 1][h],
                                                            dkacc[db], 0, 0, 0);
      };
      f32x4 l4, d4;  // row values of the current group of four scores
      auto rows = [&](auto sc, auto gc) {
        constexpr int sb = decltype(sc)::value, gq = decltype(gc)::value;
        const int r4 = sb * 32 + 8 * gq + 4 * hl;
        l4 = *(const f32x4*)(sL + r4);
        d4 = *(const f32x4*)(sDl + r4);
      };
      auto elem = [&](auto sc, auto ic) {  // score i of the lane: P and dA (unmasked)
        constexpr int sb = decltype(sc)::value, i = decltype(ic)::value;
        constexpr int e = i & 3;
        const int qi = q0 + sb * 32 + 8 * (i >> 2) + 4 * hl + e;
        float dfac;
        const float f = score_f<SCORE>(a, sa[sb & 1][i], qi, kj, slope, dfac);
        const float p = fast_exp2(fmaf(f, kLog2e, -l4[e]));
        float dA = p * (da[sb & 1][i] - d4[e]);
        if constexpr (SCORE & FA_SCORE_SOFTCAP) dA *= dfac;
        pb[sb & 1][i >> 3][i & 7] = (__bf16)p;
        dsb[sb & 1][i >> 3][i & 7] = (__bf16)dA;
      };
      auto mask_sub = [&](auto sc) {  // partial tiles: masked pairs get P = dA = 0
        constexpr int sb = decltype(sc)::value;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int r4 = sb * 32 + 8 * gq + 4 * hl;
          const i32x4 c4 = *(const i32x4*)(sDoc + r4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * gq + e;
            if (!pair_ok(pm, q0 + r4 + e, kj, c4[e], kdoc)) {
              pb[sb & 1][i >> 3][i & 7] = (__bf16)0.0f;
              dsb[sb & 1][i >> 3][i & 7] = (__bf16)0.0f;
            }
          }
        }
      };
      bwd_static_for<8>([&](auto kc) { sdp(std::integral_constant<int, 0>{}, kc); });
      bwd_static_for<QR / 32>([&](auto sc) {
        constexpr int sb = decltype(sc)::value;
        constexpr bool PREV = sb > 0, NEXT = sb + 1 < QR / 32;
        __builtin_amdgcn_sched_barrier(0);
        bwd_static_for<16>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr ((i & 3) == 0) rows(sc, std::integral_constant<int, i / 4>{});
          if constexpr ((i & 1) == 0) {
            if constexpr (PREV) dkv(std::integral_constant<int, sb - 1>{}, std::integral_constant<int, i / 2>{});
          } else {
            if constexpr (NEXT) sdp(std::integral_constant<int, sb + 1>{}, std::integral_constant<int, i / 2>{});
          }
          elem(sc, ic);
          __builtin_amdgcn_sched_barrier(0);
        });
        if (masked) mask_sub(sc);
      });
      bwd_static_for<8>([&](auto jc) { dkv(std::integral_constant<int, QR / 32 - 1>{}, jc); });
    }
  }

  // dK and dV rows go out through LDS, as in the dQ kernel: wave w stages its 32 dK rows at
  // sQ + 8 KB w and its 32 dV rows at sO + 8 KB w (after a barrier: the last step's tiles may
  // still be read by other waves), and reads back only its own rows, 4 whole rows per store.
  __syncthreads();
  {
    unsigned char* const kb8 = sQ + wave * (32 * 256);
    unsigned char* const vb8 = sO + wave * (32 * 256);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = (__bf16)(dkacc[db][gq * 4 + e] * a.sm_scale);
          v4[e] = (__bf16)dvacc[db][gq * 4 + e];
        }
        *(bf16x4*)(kb8 + tile_off(lq, db * 4 + gq) + hl * 8) = k4;
        *(bf16x4*)(vb8 + tile_off(lq, db * 4 + gq) + hl * 8) = v4;
      }
    }
    __bf16* const kop0 = (__bf16*)a.dk + b * a.dk_sb + hkv * a.dk_sh;
    __bf16* const vop0 = (__bf16*)a.dv + b * a.dv_sb + hkv * a.dv_sh;
    const int kw0 = kb * 128 + wave * 32;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4), ch = lane & 15;
      const bf16x8 k8 = *(const bf16x8*)(kb8 + tile_off(r, ch));
      const bf16x8 v8 = *(const bf16x8*)(vb8 + tile_off(r, ch));
      if (kw0 + r < a.Lkv) {
        *(bf16x8*)(kop0 + (int64_t)(kw0 + r) * a.dk_sl + ch * 8) = k8;
        *(bf16x8*)(vop0 + (int64_t)(kw0 + r) * a.dv_sl + ch * 8) = v8;
      }
    }
  }
}

// dslopes[h] = sum over batches and query blocks of the partial sums (one workgroup per head).
__global__ __launch_bounds__(256) void bwd_slope_kernel(BwdArgs a) {
  __shared__ float sRed[4];
  const int hq = blockIdx.x;
  float acc = 0.f;
  const int n = a.B * a.nqb;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int b = i / a.nqb, qb = i % a.nqb;
    acc += a.slope_part[((int64_t)b * a.Hq + hq) * a.nqb + qb];
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) sRed[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.dslopes[hq] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
}

// Column lists of a BlockMask: one wave per (mask row, kv block). Lane l tests q blocks
// c + l; membership in the ascending row lists is a binary search; ballots keep the output
// ascending.
__global__ __launch_bounds__(256) void bm_transpose_kernel(TransposeArgs t) {
  const int lane = threadIdx.x & 63;
  const int64_t col = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= (int64_t)t.Bm * t.Hm * t.nkvb) return;  // whole waves
  const int kb = (int)(col % t.nkvb);
  const int64_t mrow = col / t.nkvb;  // bm * Hm + hm
  auto find = [&](const int* lst, int n, int key) {
    int lo = 0, hi = n;  // first index with lst[i] >= key
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (lst[mid] < key) lo = mid + 1; else hi = mid;
    }
    return lo < n && lst[lo] == key;
  };
  int* qi_out = t.q_idx + col * t.nqb;
  int* fq_out = t.fullq_idx + col * t.nqb;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int np = 0, nf = 0;
  for (int c = 0; c < t.nqb; c += 64) {
    const int qb = c + lane;
    int cls = 0;
    if (qb < t.nqb) {
      const int64_t r = mrow * t.nqb + qb;
      if (find(t.kv_idx + r * t.nkvb, clamp_count(t.kv_num[r], t.nkvb), kb)) cls = 1;
      else if (find(t.full_idx + r * t.nkvb, clamp_count(t.full_num[r], t.nkvb), kb)) cls = 2;
    }
    const unsigned long long mp = __ballot(cls == 1), mf = __ballot(cls == 2);
    if (cls == 1) qi_out[np + __popcll(mp & lt)] = qb;
    if (cls == 2) fq_out[nf + __popcll(mf & lt)] = qb;
    np += __popcll(mp);
    nf += __popcll(mf);
  }
  for (int e = np + lane; e < t.nqb; e += 64) qi_out[e] = 0;
  for (int e = nf + lane; e < t.nqb; e += 64) fq_out[e] = 0;
  if (lane == 0) {
    t.q_num[col] = np;
    t.fullq_num[col] = nf;
  }
}

template <int SCORE>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  // With no query rows, only dk / dv (zeros) and dslopes (zeros) are written.
  // The dQ pass writes each row's delta and lse2, which the dK/dV pass reads: same stream, in
  // this order.
  const int64_t nq = (int64_t)a.B * a.Hq * a.nqb;
  if (nq > 0) hipLaunchKernelGGL((bwd_dq_kernel<SCORE>), dim3((unsigned)nq), dim3(256), 0, stream, a);
  const int64_t nk = (int64_t)a.B * a.Hkv * a.nkvb;
  if (nk > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<SCORE>), dim3((unsigned)nk), dim3(256), 0, stream, a);
  if ((SCORE & FA_SCORE_ALIBI) && a.dslopes)
    hipLaunchKernelGGL(bwd_slope_kernel, dim3(a.Hq), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int score, hipStream_t stream) {
  switch (score) {
    case 0: return launch_bwd_t<0>(a, stream);
    case FA_SCORE_ALIBI: return launch_bwd_t<FA_SCORE_ALIBI>(a, stream);
    case FA_SCORE_SOFTCAP: return launch_bwd_t<FA_SCORE_SOFTCAP>(a, stream);
    default: return launch_bwd_t<FA_SCORE_ALIBI | FA_SCORE_SOFTCAP>(a, stream);
  }
}

hipError_t launch_block_mask_transpose(const TransposeArgs& t, hipStream_t stream) {
  const int64_t cols = (int64_t)t.Bm * t.Hm * t.nkvb;
  if (cols == 0) return hipSuccess;
  hipLaunchKernelGGL(bm_transpose_kernel, dim3((unsigned)((cols + 3) / 4)), dim3(256), 0, stream, t);
  return hipGetLastError();
}

}  // namespace fa

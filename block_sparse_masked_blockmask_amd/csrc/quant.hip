// Quantized attention form (gfx950): int8 Q.K^T and OCP E4M3 P.V with bf16 output.
//
// FlashRT-Structures PR #1 ("LTX-2.5 attention forms"): the sage2 form runs Q.K^T on int8 and
// P.V on fp8 with bf16 output; masked sites are refused. Granularity and rounding here:
//   Q, K: one float32 scale per (batch, head, 128-token block), scale = amax / 127, code =
//         round-to-nearest-even(x / scale) clamped to +-127 (amax 0: scale 0, codes 0);
//   V:    one float32 scale per (batch, head, channel) over all tokens, scale = amax / 448, code
//         = E4M3(x / scale), round-to-nearest-even; the quotient is clamped to +-448 first
//         because the conversion instruction does not saturate (it returns NaN above 464);
//   P:    the softmax numerators P in [0, 1] are coded as E4M3(448 P); the row sum uses the
//         unrounded P; out = (sum_j P8_j V8_j) * scale_V / (448 * l).
// The forward computes S^T = K8 Q8^T on v_mfma_i32_32x32x32_i8 (exact integer dot products,
// then times scale_Q * scale_K * sm_scale) and O^T += V8^T P8^T on the 32x32x64 fp8 MFMA.
#include <hip/hip_runtime.h>

#include <cfloat>

#include <climits>

#include "device_common.h"
#include "launch.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kE4M3Max = 448.0f;
constexpr float kLog2E4M3Max = 8.807354922057604f;  // log2(448)
constexpr int kMeanRows = 1024;  // rows per partial sum of the K mean

__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

__device__ __forceinline__ float block_max_256(float x, float* s_red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_red[wave] = x;
  __syncthreads();
  x = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  return x;
}

}  // namespace

// One workgroup per (128-token block, head, batch) of Q or K: absmax scales and int8 codes, with
// one scale per 128 tokens or per 32 tokens (qk_block). With K centering, K is quantized as
// K - mean (one float32 subtraction per element, mean from quant_k_mean_*), and the Q pass also
// writes q . mean of its kv head per row.
__global__ __launch_bounds__(256) void quant_qk_kernel(QuantArgs a, int which) {
  const QuantTensor& src = which == 0 ? a.q : a.k;
  const QuantOut& dst = which == 0 ? a.q8 : a.k8;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  __shared__ float s_red[4][4];
  const int tid = threadIdx.x;
  const int r0 = blk * 128;
  const int rows = min(128, src.L - r0);
  const bool fine = a.qk_block == 32;
  // Thread t handles rows t/16 + 16*i (i = 0..7; 32-token sub-block i/2) and channels
  // 8*(t%16) .. +8.
  const unsigned short* base = src.data + b * src.sb + h * src.sh;
  const int c0 = 8 * (tid % 16);
  float mu[8];
  const float* mean_kv = nullptr;
  if (a.k_mean) {
    const int hkv = which == 0 ? h / (a.q.H / a.k.H) : h;
    mean_kv = a.k_mean + ((int64_t)b * a.k.H + hkv) * 128;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = (which == 1 && mean_kv) ? mean_kv[c0 + e] : 0.f;
  float x[8][8];
  float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = tid / 16 + 16 * i;
    if (r < rows) {
      const i32x4 raw = *(const i32x4*)(base + (int64_t)(r0 + r) * src.sl + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[i][2 * e] = bf16_to_f32((unsigned short)(raw[e] & 0xffff)) - mu[2 * e];
        x[i][2 * e + 1] = bf16_to_f32((unsigned short)((unsigned)raw[e] >> 16)) - mu[2 * e + 1];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) am[i >> 1] = fmaxf(am[i >> 1], fabsf(x[i][e]));
  }
  // Block maxima of the four 32-row sub-blocks (and of the whole block).
  const int wave = tid >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am[j] = fmaxf(am[j], __shfl_xor(am[j], o, 64));
    if ((tid & 63) == 0) s_red[wave][j] = am[j];
  }
  __syncthreads();
  float scale[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    am[j] = fmaxf(fmaxf(s_red[0][j], s_red[1][j]), fmaxf(s_red[2][j], s_red[3][j]));
  if (fine) {
#pragma unroll
    for (int j = 0; j < 4; ++j) scale[j] = am[j] / 127.0f;  // correctly rounded division
    if (tid < 4 && 32 * tid < rows) dst.scale[((int64_t)b * src.H + h) * dst.nblocks + blk * 4 + tid] = scale[tid];
  } else {
    const float s1 = fmaxf(fmaxf(am[0], am[1]), fmaxf(am[2], am[3])) / 127.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) scale[j] = s1;
    if (tid == 0) dst.scale[((int64_t)b * src.H + h) * dst.nblocks + blk] = s1;
  }
  signed char* out = dst.data + b * dst.sb + h * dst.sh;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = tid / 16 + 16 * i;
    if (r >= rows) continue;
    const float sc = scale[i >> 1];
    unsigned lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int c = 0;
      if (sc > 0.f) c = (int)fminf(fmaxf(rintf(x[i][e] / sc), -127.f), 127.f);
      const unsigned byte = (unsigned)(c & 0xff);
      if (e < 4) lo |= byte << (8 * e); else hi |= byte << (8 * (e - 4));
    }
    *(i32x2*)(out + (int64_t)(r0 + r) * dst.sl + c0) = i32x2{(int)lo, (int)hi};
  }
  if (which == 0 && a.q_delta && mean_kv) {
    // q . mean per row: 8 channels per thread, then the 16 threads of the row (lanes l ^ 1..8).
    float mk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mk[e] = mean_kv[c0 + e];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = tid / 16 + 16 * i;
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(x[i][e], mk[e], d);
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
      if ((tid & 15) == 0 && r < rows) a.q_delta[((int64_t)b * src.H + h) * src.L + r0 + r] = d;
    }
  }
}

// K centering, pass 1: per (chunk of rows, head, batch), fp64 sums of each channel over the
// chunk (bf16 values, so the sums are exact while they fit 53 bits), written to mean_part.
__global__ __launch_bounds__(256) void quant_k_mean_part_kernel(QuantArgs a, int rows_per_wg) {
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  __shared__ double s_part[16][128];
  const unsigned short* base = a.k.data + b * a.k.sb + h * a.k.sh;
  const int r_begin = chunk * rows_per_wg, r_end = min(a.k.L, r_begin + rows_per_wg);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r_begin + tid / 16; r < r_end; r += 16) {
    const i32x4 raw = *(const i32x4*)(base + (int64_t)r * a.k.sl + 8 * (tid % 16));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_to_f32((unsigned short)(raw[e] & 0xffff));
      acc[2 * e + 1] += (double)bf16_to_f32((unsigned short)((unsigned)raw[e] >> 16));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_part[tid / 16][8 * (tid % 16) + e] = acc[e];
  __syncthreads();
  if (tid < 128) {
    double sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += s_part[i][tid];
    a.mean_part[(((int64_t)b * a.k.H + h) * a.mean_chunks + chunk) * 128 + tid] = sum;
  }
}

// K centering, pass 2: mean = (sum of the partial sums, in chunk order) / L, rounded to float32.
__global__ __launch_bounds__(128) void quant_k_mean_final_kernel(QuantArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const double* part = a.mean_part + ((int64_t)b * a.k.H + h) * a.mean_chunks * 128;
  double sum = 0;
  for (int i = 0; i < a.mean_chunks; ++i) sum += part[(int64_t)i * 128 + c];
  a.k_mean[((int64_t)b * a.k.H + h) * 128 + c] = a.k.L > 0 ? (float)(sum / (double)a.k.L) : 0.f;
}

__global__ __launch_bounds__(256) void quant_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// Pass 1 for V: per-channel maximum of |x| over a chunk of rows, folded into the scale array
// as amax / 448 with an atomic max on the (non-negative) float bits. Rounding x -> x / 448 is
// monotone, so the maximum of the rounded quotients is the rounded quotient of the maximum.
__global__ __launch_bounds__(256) void quant_v_amax_kernel(QuantArgs a, int rows_per_wg) {
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  __shared__ float s_part[16][128];
  const unsigned short* base = a.v.data + b * a.v.sb + h * a.v.sh;
  const int r_begin = chunk * rows_per_wg, r_end = min(a.v.L, r_begin + rows_per_wg);
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = r_begin + tid / 16; r < r_end; r += 16) {
    const i32x4 raw = *(const i32x4*)(base + (int64_t)r * a.v.sl + 8 * (tid % 16));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[2 * e] = fmaxf(m[2 * e], fabsf(bf16_to_f32((unsigned short)(raw[e] & 0xffff))));
      m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(bf16_to_f32((unsigned short)((unsigned)raw[e] >> 16))));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_part[tid / 16][8 * (tid % 16) + e] = m[e];
  __syncthreads();
  if (tid < 128) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_part[i][tid]);
    const float sc = mx / kE4M3Max;
    atomicMax((unsigned int*)(a.v8.scale + ((int64_t)b * a.v.H + h) * 128 + tid), __float_as_uint(sc));
  }
}

// Pass 2 for V: E4M3 codes of x / scale (scale 0: code 0).
__global__ __launch_bounds__(256) void quant_v_encode_kernel(QuantArgs a, int rows_per_wg) {
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const unsigned short* base = a.v.data + b * a.v.sb + h * a.v.sh;
  unsigned char* out = (unsigned char*)a.v8.data + b * a.v8.sb + h * a.v8.sh;
  const float* sc = a.v8.scale + ((int64_t)b * a.v.H + h) * 128 + 8 * (tid % 16);
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = sc[e];
  const int r_begin = chunk * rows_per_wg, r_end = min(a.v.L, r_begin + rows_per_wg);
  for (int r = r_begin + tid / 16; r < r_end; r += 16) {
    const i32x4 raw = *(const i32x4*)(base + (int64_t)r * a.v.sl + 8 * (tid % 16));
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] = bf16_to_f32((unsigned short)(raw[e] & 0xffff));
      y[2 * e + 1] = bf16_to_f32((unsigned short)((unsigned)raw[e] >> 16));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = s[e] > 0.f ? fminf(fmaxf(y[e] / s[e], -kE4M3Max), kE4M3Max) : 0.f;
    int w0 = 0, w1 = 0;
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], w1, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
    *(i32x2*)(out + (int64_t)r * a.v8.sl + 8 * (tid % 16)) = i32x2{w0, w1};
  }
}

int quant_mean_chunks(int L) { return (L + kMeanRows - 1) / kMeanRows; }

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  const int qb = (a.q.L + 127) / 128, kb = (a.k.L + 127) / 128;
  if (a.k_mean && a.k.B > 0) {  // centering: the mean first (the Q and K passes read it)
    if (a.mean_chunks > 0)
      hipLaunchKernelGGL(quant_k_mean_part_kernel, dim3(a.mean_chunks, a.k.H, a.k.B), dim3(256), 0, stream, a,
                         kMeanRows);
    hipLaunchKernelGGL(quant_k_mean_final_kernel, dim3(a.k.H, a.k.B), dim3(128), 0, stream, a);
  }
  if (a.q.B > 0 && qb > 0)
    hipLaunchKernelGGL(quant_qk_kernel, dim3(qb, a.q.H, a.q.B), dim3(256), 0, stream, a, 0);
  if (a.k.B > 0 && kb > 0)
    hipLaunchKernelGGL(quant_qk_kernel, dim3(kb, a.k.H, a.k.B), dim3(256), 0, stream, a, 1);
  const int nscale = a.v.B * a.v.H * 128;
  if (nscale > 0) {
    hipLaunchKernelGGL(quant_zero_kernel, dim3((nscale + 255) / 256), dim3(256), 0, stream, a.v8.scale, nscale);
    if (a.v.L > 0) {
      const int rows_per_wg = 512;
      const int chunks = (a.v.L + rows_per_wg - 1) / rows_per_wg;
      hipLaunchKernelGGL(quant_v_amax_kernel, dim3(chunks, a.v.H, a.v.B), dim3(256), 0, stream, a, rows_per_wg);
      hipLaunchKernelGGL(quant_v_encode_kernel, dim3(chunks, a.v.H, a.v.B), dim3(256), 0, stream, a, rows_per_wg);
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Quantized forward. One workgroup of 4 waves per (batch, query head, 128-query block); wave w
// owns 32 queries, as in the bf16 kernel. Keys in steps of 64: the int8 K rows and fp8 V rows
// of a step (8 KB each) stream into a ring of kQBuf LDS buffers with global_load_lds_dwordx4,
// kQBuf - 1 steps ahead of the step being computed (64 KB of LDS, two workgroups per CU). A step's
// int8 and fp8 products take half the time of the bf16 ones, so one step of lead time left each
// step waiting for its transfers.
//
// LDS rows are 128 bytes (8 chunks of 16); chunk c of row r is stored at position c ^ ((r/2)%8),
// which spreads 16 consecutive rows read at one chunk over distinct banks. V rows are stored
// in a permuted order within each 16-row group (logical rows 0-3, 8-11, 4-7, 12-15), so that the
// 8 consecutive physical rows returned by one ds_read_b64_tr_b8 are exactly the keys of one lane
// half's softmax numerators, in accumulator order.
// ---------------------------------------------------------------------------------------------
namespace {

constexpr int kQStep = 64;
constexpr int kQStepBytes = kQStep * 128;
constexpr int kQBuf = 4;  // LDS ring buffers (steps in flight: kQBuf - 1)

// Each buffer is a distinct LDS object named at compile time, so that the compiler does not wait
// for the transfers into the other buffers before reading one.
__shared__ __attribute__((aligned(1024))) unsigned char q_k0[kQStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char q_v0[kQStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char q_k1[kQStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char q_v1[kQStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char q_k2[kQStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char q_v2[kQStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char q_k3[kQStepBytes];
__shared__ __attribute__((aligned(1024))) unsigned char q_v3[kQStepBytes];

template <int B> __device__ __forceinline__ unsigned char* qkbuf() {
  return B == 0 ? q_k0 : B == 1 ? q_k1 : B == 2 ? q_k2 : q_k3;
}
template <int B> __device__ __forceinline__ unsigned char* qvbuf() {
  return B == 0 ? q_v0 : B == 1 ? q_v1 : B == 2 ? q_v2 : q_v3;
}

__device__ __forceinline__ int qswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int qoff(int r, int chunk) { return r * 128 + ((chunk ^ qswz(r)) << 4); }
// Logical row of physical row p within a 16-row group: 0-3, 8-11, 4-7, 12-15.
__device__ __forceinline__ int vperm(int p) { return (p & ~15) | ((p & 3) | ((p & 4) << 1) | ((p & 8) >> 1)); }

__device__ __forceinline__ void qdma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
// The compiler does not track the LDS writes of global_load_lds: wait for them explicitly, with at
// most N vector-memory operations of this wave still outstanding.
template <int N> __device__ __forceinline__ void qwait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier without the memory fence of __syncthreads(): that fence makes the compiler
// wait for every outstanding transfer into LDS (vmcnt(0)), including the ones for later steps.
// Each wave has waited for its own transfers of the step explicitly, and its LDS reads of the
// previous step have returned before their products; the empty asm statements keep the compiler
// from moving LDS accesses or transfers across the barrier.
__device__ __forceinline__ void qbarrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct QCtx {
  int wave, lane, hl, lq, g16, s16, qi;
  bool q_in;
  const signed char* kp;
  const unsigned char* vp;
  const float* ks;   // K block scales of this (b, hkv)
  float qscale;      // scale_Q * sm_scale * log2(e)
  int koff, voff;    // byte offsets of this lane's first K and V transfer chunks from a step's row 0
  // Byte offsets in a step buffer of this lane's first K-operand read (row lq, chunk hl) and first
  // transposed V read; the others follow by XOR and add (the swizzle's fields are disjoint bit
  // ranges): K sub-block nb, k-step ks at (kx0 ^ 32 ks) + 4096 nb; V channel block db, row group rr
  // at (vx0 ^ 32 db) + 2048 rr.
  int kx0, vx0;
};

struct QState {
  f32x16 oacc[4];
  float m_run, l_run;
};

template <int B>
__device__ __forceinline__ void qissue(const QuantFwdArgs& a, const QCtx& c, int kv0) {
  // 8 KB per tensor = 8 segments of 1 KB (8 rows); wave w loads segments w and w + 4, physical rows
  // 8 w + lane / 8 and 32 more. The chunk swizzle and the V row order repeat every 16 rows, so the
  // second segment's lane offsets are the first's plus 32 rows: a step inside the keys needs only
  // the uniform row address and the lane's constant offsets.
  if (kv0 + kQStep <= a.Lkv) {
    const signed char* kb = c.kp + (int64_t)kv0 * a.k_sl;
    const unsigned char* vb = c.vp + (int64_t)kv0 * a.v_sl;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = i * 4 + c.wave;
      qdma16(kb + (int64_t)(32 * i) * a.k_sl + c.koff, qkbuf<B>() + seg * 1024);
      qdma16(vb + (int64_t)(32 * i) * a.v_sl + c.voff, qvbuf<B>() + seg * 1024);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = i * 4 + c.wave;
      const int p = seg * 8 + (c.lane >> 3);  // physical row written by this lane
      const int pos = c.lane & 7;             // physical chunk position
      const int kr = min(kv0 + p, a.Lkv - 1);
      const int vr = min(kv0 + vperm(p), a.Lkv - 1);
      qdma16(c.kp + (int64_t)kr * a.k_sl + ((pos ^ qswz(p)) << 4), qkbuf<B>() + seg * 1024);
      qdma16(c.vp + (int64_t)vr * a.v_sl + ((pos ^ qswz(p)) << 4), qvbuf<B>() + seg * 1024);
    }
  }
}

// RAGGED: the step reaches past the last key (only the last step can), so scores of keys past
// it are set to -inf; other steps skip that test. The numerators are produced already scaled by
// 448: exp2(t - (m - log2 448)) = 448 P, which is the E4M3 code's input; the running sum l_run
// therefore holds 448 times the row sum (the epilogue divides by it as it stands).
template <int B, bool RAGGED>
__device__ __forceinline__ void qcompute(const QuantFwdArgs& a, const QCtx& c, const i32x4 (&qreg)[4], QState& st,
                                         int kv0, float2 kscale) {
  const unsigned char* sK = qkbuf<B>();
  const unsigned char* sV = qvbuf<B>();
  // Re-defined here (no instruction is emitted) so that the compiler forms buffer + offset inside
  // the step, where the buffer address folds into the instruction's immediate offset, instead of
  // keeping one hoisted register per buffer and read.
  int kx0 = c.kx0, vx0 = c.vx0;
  asm volatile("" : "+v"(kx0), "+v"(vx0));
  // S^T = K8 Q8^T: exact int32 dot products, 4 k-steps of 32 channels per 32-key sub-block.
  i32x16 iacc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    iacc[nb] = i32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const i32x4 kf = *(const i32x4*)(sK + nb * 4096 + (kx0 ^ (32 * ks)));
      iacc[nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qreg[ks], iacc[nb], 0, 0, 0);
    }
  }
  // Per 32-key sub-block: the log2-domain score of a product is its value times the sub-block's
  // scale. The row maximum is taken on the products of each sub-block and scaled once (rounding is
  // monotone, so this is the maximum of the rounded scores); the exponent below applies the scale
  // in its FMA. A zero scale (an all-zero block) is raised to the smallest normal float, so that a
  // masked product (-inf) stays -inf instead of giving -inf * 0; the scores it gives (at most
  // 2^21 times that) are zero to fp32 precision once the maximum is subtracted.
  const float scs[2] = {fmaxf(c.qscale * kscale.x, FLT_MIN), fmaxf(c.qscale * kscale.y, FLT_MIN)};
  float t[2][16];
  float mxs[2] = {-INFINITY, -INFINITY};
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kv = kv0 + nb * 32 + (i >> 2) * 8 + c.hl * 4 + (i & 3);
      t[nb][i] = (!RAGGED || kv < a.Lkv) ? (float)iacc[nb][i] : -INFINITY;
      mxs[nb] = fmaxf(mxs[nb], t[nb][i]);
    }
  }
  float mx = half_swap_max(fmaxf(mxs[0] * scs[0], mxs[1] * scs[1]));
  // Exact running maximum (P <= 1 keeps 448 P inside the E4M3 range).
  const float m_new = fmaxf(st.m_run, mx);
  const bool raise = m_new > st.m_run;
  // The numerators and P.V products follow in two copies, one per outcome of the rescale test:
  // with one copy after a conditional rescale, the compiler kept O in two register sets and copied
  // all 64 accumulators on every step.
  auto finish = [&]() {
  // P^T as the fp8 B operand: byte j of the 32 holds key position (j / 16, element j % 16).
  // 448 P <= 448 up to the exponential's last-place error, far below 464, where the conversion
  // stops rounding to 448.
  const float m448 = st.m_run - kLog2E4M3Max;
  i32x8 pb;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int nb = w >> 2, i0 = (w & 3) * 4;
    const float p0 = fast_exp2(fmaf(t[nb][i0], scs[nb], -m448));
    const float p1 = fast_exp2(fmaf(t[nb][i0 + 1], scs[nb], -m448));
    const float p2 = fast_exp2(fmaf(t[nb][i0 + 2], scs[nb], -m448));
    const float p3 = fast_exp2(fmaf(t[nb][i0 + 3], scs[nb], -m448));
    st.l_run += (p0 + p1) + (p2 + p3);
    int word = 0;
    word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, word, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
    pb[w] = word;
  }
  // O^T += V8^T P8^T. Transposed reads: in each 16-lane group, source lane s points at physical
  // row base + s/2 and channels d0 + 8*(s%2); lane i receives channel d0 + i of rows base..+7.
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    i32x8 vf;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sV + rr * 2048 + (vx0 ^ (32 * db))));
      vf[2 * rr] = v2[0];
      vf[2 * rr + 1] = v2[1];
    }
    // Formats 0/0: both operands E4M3; scale exponents 127 mean a factor of 1.
    st.oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pb, st.oacc[db], 0, 0, 0, 127, 0, 127);
  }
  };
  if (__builtin_amdgcn_readfirstlane(__ballot(raise) != 0)) {
    const float alpha = raise ? fast_exp2(st.m_run - m_new) : 1.0f;
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.oacc[db] *= alpha;
    st.m_run = m_new;
    finish();
  } else {
    finish();
  }
}

}  // namespace

// QKB: tokens per Q/K scale (128 or 32).
template <int QKB>
__global__ __launch_bounds__(256, 2) void fwd_quant_kernel(QuantFwdArgs a) {
  int w = xcd_remap(blockIdx.x, a.total_wg);
  const int g = w % a.group;
  w /= a.group;
  const int qb = a.nqw - 1 - (w % a.nqw);
  w /= a.nqw;
  const int hkv = w % a.Hkv, b = w / a.Hkv;
  const int hq = hkv * a.group + g;

  QCtx c;
  c.wave = threadIdx.x >> 6;
  c.lane = threadIdx.x & 63;
  c.hl = c.lane >> 5;
  c.lq = c.lane & 31;
  c.g16 = c.lane >> 4;
  c.s16 = c.lane & 15;
  c.qi = qb * 128 + c.wave * 32 + c.lq;
  c.q_in = c.qi < a.Lq;
  c.kp = a.k + b * a.k_sb + hkv * a.k_sh;
  c.vp = a.v + b * a.v_sb + hkv * a.v_sh;
  c.ks = a.k_scale + ((int64_t)b * a.Hkv + hkv) * a.nkb;
  {
    const int p0 = c.wave * 8 + (c.lane >> 3), ch = ((c.lane & 7) ^ qswz(p0)) << 4;
    c.koff = p0 * (int)a.k_sl + ch;
    c.voff = vperm(p0) * (int)a.v_sl + ch;
  }
  c.kx0 = qoff(c.lq, c.hl);
  {
    const int d0 = 16 * (c.g16 & 1) + 8 * (c.s16 & 1);
    c.vx0 = qoff((c.g16 >> 1) * 8 + (c.s16 >> 1), d0 >> 4) + (d0 & 15);
  }
  // Q scale of this wave's 32 queries: one per 128-query block, or one per wave (32-token
  // blocks); a wave past the end reads the last block's scale (its rows are not written).
  const int qsb = QKB == 32 ? min(qb * 4 + c.wave, a.nqb - 1) : qb;
  c.qscale = a.q_scale[((int64_t)b * a.Hq + hq) * a.nqb + qsb] * a.scale_log2;

  const int nsteps = (a.Lkv + kQStep - 1) / kQStep;
  // K scales of step s for its two 32-key sub-blocks: a 64-key step lies inside one 128-key
  // block; with 32-token blocks each sub-block has its own (past the end: the last one, whose
  // keys are masked). Each step's scales are loaded with its transfers, so that their wait is the
  // step's own.
  // Read through the constant address space (the scales do not change during the kernel): with a
  // uniform address these are scalar loads, which the vector-memory waits of the steps do not
  // count, and the values stay in scalar registers.
  const __attribute__((address_space(4))) float* ksv = (const __attribute__((address_space(4))) float*)c.ks;
  auto kscales = [&](int kv0) {
    if constexpr (QKB == 32) {
      const int i0 = kv0 >> 5;
      const float x = ksv[i0];
      const float y = ksv[min(i0 + 1, a.nkb - 1)];
      return make_float2(x, y);
    }
    const float x = ksv[kv0 >> 7];
    return make_float2(x, x);
  };
  constexpr int OPS = 4;  // vector-memory operations per lane and step (the transfers)
  static_assert(kQBuf == 4, "the prologue and the step loop below are written for four buffers");

  // Q8^T as the int8 B operand: lane holds Q8[qi][32*ks + 16*hl .. +16] for ks = 0..3. Loaded
  // before the prologue's transfers, so that it is in when the first step's are.
  const signed char* qp = a.q + b * a.q_sb + hq * a.q_sh;
  i32x4 qreg[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qreg[ks] = c.q_in ? *(const i32x4*)(qp + (int64_t)c.qi * a.q_sl + ks * 32 + c.hl * 16) : i32x4{};

  // Prologue: steps 0 .. kQBuf-2 in flight.
  float2 ks_ring[kQBuf];
#pragma unroll
  for (int j = 0; j < kQBuf; ++j) ks_ring[j] = make_float2(0.f, 0.f);
  if (nsteps > 0) { qissue<0>(a, c, 0); ks_ring[0] = kscales(0); }
  if (nsteps > 1) { qissue<1>(a, c, kQStep); ks_ring[1] = kscales(kQStep); }
  if (nsteps > 2) { qissue<2>(a, c, 2 * kQStep); ks_ring[2] = kscales(2 * kQStep); }


  QState st;
#pragma unroll
  for (int db = 0; db < 4; ++db) st.oacc[db] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  // Step s: wait for its transfers (the kQBuf - 2 later steps' may stay in flight; near the end,
  // where fewer were issued, for all), make sure every wave is done with the buffer about to be
  // refilled (step s - 1's), refill it with step s + kQBuf - 1, compute.
  auto step = [&](auto bufc, int s) {
    constexpr int B = decltype(bufc)::value;
    constexpr int NB = (B + kQBuf - 1) % kQBuf;
    if (s + kQBuf - 2 < nsteps) qwait_vmem<(kQBuf - 2) * OPS>();
    else qwait_vmem<0>();
    qbarrier();
    const int sn = s + kQBuf - 1;
    if (sn < nsteps) {
      qissue<NB>(a, c, sn * kQStep);
      ks_ring[NB] = kscales(sn * kQStep);
    }
    if ((s + 1) * kQStep <= a.Lkv) qcompute<B, false>(a, c, qreg, st, s * kQStep, ks_ring[B]);
    else qcompute<B, true>(a, c, qreg, st, s * kQStep, ks_ring[B]);
  };
  for (int s = 0; s < nsteps; s += kQBuf) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 < nsteps) step(std::integral_constant<int, 1>{}, s + 1);
    if (s + 2 < nsteps) step(std::integral_constant<int, 2>{}, s + 2);
    if (s + 3 < nsteps) step(std::integral_constant<int, 3>{}, s + 3);
  }
  qwait_vmem<0>();  // no transfer may outlive the workgroup's LDS

  // Epilogue: out = O * scale_V[channel] / (448 l), bf16 (l_tot is already 448 l); lse in
  // natural log.
  const float l_tot = half_swap_sum(st.l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (c.q_in) {
    const float* vs = a.v_scale + ((int64_t)b * a.Hkv + hkv) * 128;
    __bf16* op = a.o + b * a.o_sb + hq * a.o_sh + (int64_t)c.qi * a.o_sl;
    // All channel scales first: interleaved with the stores, each load waited for the one before.
    f32x4 s4[4][4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) s4[db][gq] = *(const f32x4*)(vs + db * 32 + gq * 8 + c.hl * 4);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + gq * 8 + c.hl * 4;
        bf16x4 o4;
        o4[0] = (__bf16)(st.oacc[db][gq * 4 + 0] * s4[db][gq][0] * inv);
        o4[1] = (__bf16)(st.oacc[db][gq * 4 + 1] * s4[db][gq][1] * inv);
        o4[2] = (__bf16)(st.oacc[db][gq * 4 + 2] * s4[db][gq][2] * inv);
        o4[3] = (__bf16)(st.oacc[db][gq * 4 + 3] * s4[db][gq][3] * inv);
        *(bf16x4*)(op + d) = o4;
      }
    }
    if (a.lse && c.hl == 0) {
      // With centred keys the scores are shifted by -sm_scale (q . mean): add it back.
      const int64_t row = ((int64_t)b * a.Hq + hq) * a.Lq + c.qi;
      const float corr = a.q_delta ? a.sm_scale * a.q_delta[row] : 0.f;
      a.lse[row] = l_tot > 0.f ? (st.m_run - kLog2E4M3Max + __log2f(l_tot)) * kLn2 + corr : -INFINITY;
    }
  }
}

hipError_t launch_fwd_quant(const QuantFwdArgs& a, hipStream_t stream) {
  if (a.total_wg == 0) return hipSuccess;
  if (a.qk_block == 32) hipLaunchKernelGGL(fwd_quant_kernel<32>, dim3(a.total_wg), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(fwd_quant_kernel<128>, dim3(a.total_wg), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa

// Kernel argument blocks and launchers (host side). The C-ABI layer (api.cpp) validates every
// argument and then calls these; they only enqueue work on the given stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct BlockMaskArgs {
  int flags, window, prefix_len;
  int B, Lq, Lkv, BQ, BK, nqb, nkvb, Bm;
  const int* q_doc;
  const int* kv_doc;
  int* qsum;    // [B][nqb][4] min id, max id, dense flag, 0 of each query block (DOC only)
  int* kvsum;   // [B][nkvb][4]
  int* kv_num;
  int* kv_idx;
  int* full_num;
  int* full_idx;
  int* row_order;  // [Bm][nqb] query blocks by decreasing cost, or null
  int self_ids;    // DOC with q_doc and kv_doc the same array (and Lq == Lkv)
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sh, q_sl;
  int64_t k_sb, k_sh, k_sl;
  int64_t v_sb, v_sh, v_sl;
  int64_t o_sb, o_sh, o_sl;
  int B, Hq, Hkv, Lq, Lkv, group;
  // BlockMask (all_full = 1: no BlockMask, every tile is full)
  const int* kv_num;
  const int* kv_idx;
  const int* full_num;
  const int* full_idx;
  int Bm, Hm, nqb, nkvb, all_full;
  const int* row_order;  // [Bm][Hm][nqb] schedule (query blocks by decreasing cost), or null
  // mask_mod / score_mod
  int flags, window, prefix_len;
  const int* q_doc;
  const int* kv_doc;
  float sm_scale, scale_log2, softcap, inv_softcap;
  // Folded score_mod constants (log2 domain): soft-cap input and output factors, and the
  // factor applied to each ALiBi slope.
  float sc_in, sc_out, sc_out2, slope_mul;
  const float* slopes;
  int total_wg;
  // Split-KV: nsplit > 1 cuts each work item's tile list into nsplit contiguous ranges, one
  // workgroup each; they write normalised partial outputs and their lse to part_o
  // [nsplit][B][Hq][Lq][128] (fp32) and part_lse [nsplit][B][Hq][Lq] instead of o and lse.
  int nsplit;
  float* part_o;
  float* part_lse;
  int pack;  // with nsplit > 1: one workgroup per kv head holds all (query head, query) rows
};

// Merge of split-KV partial results into o (bf16) and lse.
struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  __bf16* o;
  float* lse;
  int64_t o_sb, o_sh, o_sl;
  int B, Hq, Lq, nsplit;
};

// Backward (bf16, head dim 128). Gradients dq [B][Hq][Lq][128], dk and dv [B][Hkv][Lkv][128]
// (bf16, element strides); the workspace holds per-row lse2 = lse * log2(e) (+inf for rows with
// no allowed key, so that their probabilities come out 0) and delta = dout . out, and the
// per-(b, hq, 128-query block) partial sums of the ALiBi-slope gradient.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dslopes;
  int64_t q_sb, q_sh, q_sl;
  int64_t k_sb, k_sh, k_sl;
  int64_t v_sb, v_sh, v_sl;
  int64_t o_sb, o_sh, o_sl;
  int64_t do_sb, do_sh, do_sl;
  int64_t dq_sb, dq_sh, dq_sl;
  int64_t dk_sb, dk_sh, dk_sl;
  int64_t dv_sb, dv_sh, dv_sl;
  int B, Hq, Hkv, Lq, Lkv, group;
  // Row lists (per 128-query block) for dq, column lists (per 128-key block) for dk/dv;
  // all_full = 1: no BlockMask, every tile is full. row_order: the BlockMask's optional
  // schedule (query blocks of each row set by decreasing cost), used by the dq pass, or null.
  const int* row_order;
  const int* col_order;  // the transposed BlockMask's optional column schedule (dk/dv pass), or null
  const int* kv_num;
  const int* kv_idx;
  const int* full_num;
  const int* full_idx;
  const int* q_num;
  const int* q_idx;
  const int* fullq_num;
  const int* fullq_idx;
  int Bm, Hm, nqb, nkvb, all_full;
  int flags, window, prefix_len;
  const int* q_doc;
  const int* kv_doc;
  float sm_scale, softcap, inv_softcap;
  const float* slopes;
  float* lse2;        // [B][Hq][Lq]
  float* delta;       // [B][Hq][Lq]
  float* slope_part;  // [B][Hq][nqb], or null when no slope gradient is asked for
};

// Column view of a BlockMask (q-block lists per kv block).
struct TransposeArgs {
  int Bm, Hm, nqb, nkvb;
  const int* kv_num;
  const int* kv_idx;
  const int* full_num;
  const int* full_idx;
  int* q_num;
  int* q_idx;
  int* fullq_num;
  int* fullq_idx;
  int* col_order;  // [Bm][Hm][nkvb] columns by decreasing cost, or null
};

// Quantized form: bf16 sources and int8 / E4M3 outputs (element strides; int8 elements are bytes).
struct QuantTensor {
  const unsigned short* data;  // bf16 bit patterns
  int B, H, L;
  int64_t sb, sh, sl;
};
struct QuantOut {
  signed char* data;           // int8 codes, or E4M3 codes for V
  float* scale;                // Q/K: [B][H][nblocks]; V: [B][H][128]
  int nblocks;
  int64_t sb, sh, sl;
};
struct QuantArgs {
  QuantTensor q, k, v;
  QuantOut q8, k8, v8;
  int qk_block;        // tokens per Q/K scale: 128 or 32
  float* k_mean;       // K centering: float32 [B][Hkv][128] written (NULL: no centering)
  float* q_delta;      // with centering: q . k_mean per query row, float32 [B][Hq][Lq] (may be NULL)
  double* mean_part;   // with centering: per-chunk partial sums [B][Hkv][chunks][128]
  int mean_chunks;
};

struct QuantFwdArgs {
  const signed char* q;
  const signed char* k;
  const unsigned char* v;
  __bf16* o;
  float* lse;
  int64_t q_sb, q_sh, q_sl, k_sb, k_sh, k_sl, v_sb, v_sh, v_sl, o_sb, o_sh, o_sl;
  const float* q_scale;  // [B][Hq][nqb]
  const float* k_scale;  // [B][Hkv][nkb]
  const float* v_scale;  // [B][Hkv][128]
  int B, Hq, Hkv, Lq, Lkv, group;
  int nqb, nkb;          // Q and K scale blocks per (batch, head): ceil(L / qk_block)
  int nqw;               // 128-query work blocks per (batch, query head)
  float scale_log2;      // sm_scale * log2(e)
  int total_wg;
  int qk_block;          // tokens per Q/K scale: 128 or 32
  const float* q_delta;  // K centering: lse += sm_scale * q_delta[row] (NULL: none)
  float sm_scale;
};

hipError_t launch_block_mask(const BlockMaskArgs& a, hipStream_t stream);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
int quant_mean_chunks(int L);  // partial sums of the K mean (1024 rows each)
hipError_t launch_fwd_quant(const QuantFwdArgs& a, hipStream_t stream);
// dtype 0 = f32, 1 = bf16; q_block 128 (f32, bf16) or 256 (bf16); kv_block in {64, 128};
// score bits FA_SCORE_*.
hipError_t launch_fwd(const FwdArgs& a, int dtype, int q_block, int kv_block, int score, hipStream_t stream);
hipError_t launch_splitkv_merge(const MergeArgs& m, hipStream_t stream);
// bf16 forward with every tile full (no BlockMask), software-pipelined, 256-query blocks.
hipError_t launch_fwd_dense(const FwdArgs& a, int score, hipStream_t stream);
// bf16 block-sparse forward, software-pipelined, 128-query blocks, masks without document ids
// (nsplit 1); kv_block in {64, 128}.
hipError_t launch_fwd_pipe(const FwdArgs& a, int kv_block, int score, hipStream_t stream);
// Backward: dq (with the rows' delta and lse2, and the slope partials), dk/dv, slope reduction.
hipError_t launch_bwd(const BwdArgs& a, int score, hipStream_t stream);
hipError_t launch_block_mask_transpose(const TransposeArgs& t, hipStream_t stream);
// Sort nsets row sets of a.nqb entries by row_order_key of (a.full_num, a.kv_num) into
// a.row_order (the builder's schedule kernel, also used for the transposed BlockMask's columns).
hipError_t launch_block_mask_order(const BlockMaskArgs& a, int nsets, hipStream_t stream);

}  // namespace fa

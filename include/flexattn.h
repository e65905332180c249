/*
 * flexattn.h — C ABI of the block-sparse masked attention forward (and its backward) for MI355X
 * (gfx950).
 *
 * The operation (FlexAttention guide, "The Core Design Principles"):
 *     out_i = sum_j softmax_j( score_mod(q_i . k_j * sm_scale) restricted to mask_mod(i, j) ) v_j
 * computed tile by tile with an online softmax; tiles that the mask leaves empty are never
 * loaded, using a precomputed BlockMask (guide, "Systems Mechanics", item 1: full tiles run
 * without mask branches, empty tiles are skipped, partial tiles are masked per token).
 *
 * Because score_mod and mask_mod are user functions on that page, this ABI exposes a fixed set
 * of them as bit flags (below). All predicates use absolute token positions.
 *
 * Conventions shared by every entry point:
 *   - Every buffer is owned by the caller. The library allocates no device memory and never
 *     synchronises the host; all work is enqueued on the caller's `stream` and is asynchronous.
 *     Kernel faults surface at the caller's next synchronisation.
 *   - The device entry points enqueue kernels only (no memset, copy or allocation), so a
 *     sequence of calls can be captured in a HIP graph and replayed; a replay reads the
 *     buffers' current contents.
 *   - Device pointers must point into memory of the current HIP device.
 *   - On any status other than FA_OK nothing has been enqueued and no output has been written;
 *     flexattn_last_error() gives the reason. There is no silent fallback path.
 *   - The kernels are built for gfx950 (MI355X) only. Every entry point that enqueues work checks,
 *     after validating its arguments, that the current device is a gfx950 and otherwise returns
 *     FA_ERR_UNSUPPORTED naming the device's architecture (the FlashRT PR's convention that an
 *     unserved site is refused with its reason). The name is read once per device. The
 *     environment variable FLEXATTN_DEVICE_ARCH, when set, stands in for the device's name (it
 *     exists so that the refusal can be tested on a machine without the device).
 *   - Calls are thread safe; calls that overlap on the same output buffers race.
 */
#ifndef FLEXATTN_H
#define FLEXATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,   /* caller bug: null/misaligned pointer, shape mismatch, bad flags */
  FA_ERR_UNSUPPORTED = 2,   /* valid request outside what this library serves (reason given) */
  FA_ERR_DEVICE = 3         /* HIP reported an error while enqueuing (reason given) */
} fa_status;

typedef enum {
  FA_F32 = 0,        /* float32 */
  FA_BF16 = 1,       /* bfloat16 */
  FA_I8 = 2,         /* int8 codes with float32 scales (quantized form) */
  FA_FP8_E4M3 = 3    /* OCP E4M3 codes with float32 scales (quantized form) */
} fa_dtype;

/* mask_mod flags; the enabled predicates are ANDed (the guide's demo ANDs causal and window).
 *   DOC       q_doc[b][i] == kv_doc[b][j]   (guide, "Production Engineering" 1: document
 *             packing; also TiRex2's grouped variate attention, where packed variates of
 *             unrelated groups are masked — TiRex2 PR "perf: expose FlexAttention loader
 *             override", "Context")
 *   CAUSAL    i >= j                        (guide, "Implementation" demo)
 *   WINDOW    i - j < window                (guide demo's sliding window; strict, so the demo's
 *             "<= 512" is window = 513)
 *   PREFIX_LM j < prefix_len || i >= j      (guide, "Production Engineering" 2; it contains
 *             causal, so PREFIX_LM together with CAUSAL is rejected as FA_ERR_INVALID_ARG) */
enum { FA_MASK_NONE = 0, FA_MASK_DOC = 1, FA_MASK_CAUSAL = 2, FA_MASK_WINDOW = 4, FA_MASK_PREFIX_LM = 8 };

/* score_mod flags, applied to the scaled score s in this order:
 *   ALIBI     s - alibi_slopes[h] * |i - j|   (guide demo; h is the query head)
 *   SOFTCAP   softcap * tanh(s / softcap)     (guide, "The Problem": logit soft-capping) */
enum { FA_SCORE_NONE = 0, FA_SCORE_ALIBI = 1, FA_SCORE_SOFTCAP = 2 };

/* A [B, H, L, D] tensor in device memory; element strides, the D dimension contiguous.
 * `scale` (device, float32) is used by the quantized dtypes only and must be NULL otherwise; a
 * quantized Q or K tensor with no rows (B * L = 0) may leave it NULL, having no scales. */
typedef struct {
  void* data;
  int32_t dtype;                 /* fa_dtype */
  int32_t B, H, L, D;
  int64_t stride_b, stride_h, stride_l;
  const float* scale;
} fa_tensor;

typedef struct {
  float sm_scale;                /* <= 0 selects 1/sqrt(D) */
  int32_t window;                /* WINDOW: must be > 0 */
  int32_t prefix_len;            /* PREFIX_LM: must be >= 0 */
  float softcap;                 /* SOFTCAP: C, must be > 0 */
  const float* alibi_slopes;     /* ALIBI: float32 [Hq], device */
  const int32_t* q_doc;          /* DOC: int32 [B][Lq], device, contiguous */
  const int32_t* kv_doc;         /* DOC: int32 [B][Lkv], device, contiguous; may alias q_doc */
} fa_params;

/* BlockMask (guide, "Systems Mechanics" 1; field names as in FlexAttention's BlockMask).
 * For each mask row (bm, hm) and query block qb, the kv blocks whose tiles are partial
 * (kv_indices) and full (full_kv_indices), each list ascending with its length in the
 * matching *_num_blocks entry and the unused tail set to 0. Shapes (int32, device):
 *   kv_num_blocks, full_kv_num_blocks : [Bm][Hm][n_qb]
 *   kv_indices, full_kv_indices       : [Bm][Hm][n_qb][n_kvb]
 * n_qb = ceil(q_len / q_block), n_kvb = ceil(kv_len / kv_block). Bm is 1 (one row set for
 * every batch) or B; Hm is 1 or Hq. A tile is classified over its in-range pairs only, so a
 * ragged edge tile whose in-range pairs are all allowed is full.
 *
 * row_order (optional, int32 [Bm][Hm][n_qb], NULL when unused) is a schedule, not part of the
 * mask: for each mask row set, the query blocks sorted by decreasing estimated cost
 * 4 * full + 5 * partial live tiles, ties by increasing query block (identity order when
 * n_qb > 8192). The builders fill it when the pointer is set. When it is set, the forward
 * (and the dq pass of flexattn_bwd) starts the costliest query blocks first, so that long
 * rows (long documents under causal masks) do not finish last; results are identical with or
 * without it. A caller-written
 * row_order must be a permutation of 0..n_qb-1 in each row set (entries are clamped into
 * range; a repeated entry leaves some output rows unwritten). */
typedef struct {
  int32_t Bm, Hm, q_len, kv_len, q_block, kv_block, n_qb, n_kvb;
  int32_t* kv_num_blocks;
  int32_t* kv_indices;
  int32_t* full_kv_num_blocks;
  int32_t* full_kv_indices;
  int32_t* row_order;
} fa_block_mask;

/* Bytes of all four BlockMask arrays together (two count arrays and two index arrays, int32)
 * for the given dimensions; 0 on invalid dimensions. The optional row_order adds one count
 * array's bytes. (The FlashRT PR's caller-owned workspace convention: the caller sizes and owns
 * every buffer once per bound shape.) */
size_t flexattn_block_mask_bytes(int Bm, int Hm, int q_len, int kv_len, int q_block, int kv_block);

/* Bytes of ONE index array ([Bm][Hm][n_qb][n_kvb] int32) and of ONE count array
 * ([Bm][Hm][n_qb] int32) for the given dimensions; 0 on invalid dimensions. */
size_t flexattn_block_mask_index_bytes(int Bm, int Hm, int q_len, int kv_len, int q_block, int kv_block);
size_t flexattn_block_mask_count_bytes(int Bm, int Hm, int q_len, int q_block);

/* Device scratch needed by flexattn_block_mask_build (per-block document-id summaries when DOC
 * is set: 16 bytes per query block and per kv block and batch; else 0). */
size_t flexattn_block_mask_workspace_bytes(int mask_kind, int B, int q_len, int kv_len,
                                           int q_block, int kv_block);

/* Build a BlockMask on the device by classifying every (q block, kv block) tile as full,
 * partial or empty under mask_kind (guide, "Systems Mechanics" 1: create_block_mask evaluates
 * the mask over each block's bounding box). The caller fills `out`'s dimensions (Bm, Hm, q_len,
 * kv_len, q_block, kv_block, n_qb, n_kvb) and its four array pointers; Bm must be B when DOC is
 * set (1 or B otherwise), Hm must be 1 (no flag depends on the head). q_block is 64, 128 or
 * 256 and kv_block is 64 or 128. Reads p->q_doc / p->kv_doc (DOC), p->window (WINDOW), p->prefix_len (PREFIX_LM).
 * The arrays of `out` must be 4-byte aligned (FA_ERR_INVALID_ARG otherwise).
 * `workspace` must hold flexattn_block_mask_workspace_bytes(...) bytes, 16-byte aligned (may be
 * NULL if 0).
 * Classification is exact: the lists equal exhaustive evaluation of every in-range pair. */
fa_status flexattn_block_mask_build(int mask_kind, const fa_params* p, int B, int q_len, int kv_len,
                                    fa_block_mask* out, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Allocation-free variant of flexattn_block_mask_build, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Arguments, validation, kernels and results are those of
 * flexattn_block_mask_build; the builder's scratch (the per-block document-id summaries, 16 bytes
 * per query block and per kv block and batch, DOC only) comes from a static device array of
 * flexattn_block_mask_noalloc_max_bytes() bytes (1 MiB) that each device holds for the life of the
 * process. A request needing more is refused with FA_ERR_UNSUPPORTED before anything is enqueued.
 * The call allocates nothing (no hipMalloc, no allocating library call). Calls that overlap on
 * one device share the array and race; the caller orders them (one stream, or events). Nothing in
 * the array needs to start at zero: every summary is written before it is read. */
size_t flexattn_block_mask_noalloc_max_bytes(void);
fa_status flexattn_block_mask_build_noalloc(int mask_kind, const fa_params* p, int B, int q_len, int kv_len,
                                            fa_block_mask* out, hipStream_t stream);

/* The same BlockMask built on the host, on the calling thread: p->q_doc / p->kv_doc (DOC) and the
 * four arrays of `out` are host memory; no workspace, no stream. Validation, block sizes and
 * results are those of flexattn_block_mask_build (exact classification; the two builders share
 * their closed forms). For callers whose document ids live on the host, or that build a mask
 * once and upload it. */
fa_status flexattn_block_mask_build_host(int mask_kind, const fa_params* p, int B, int q_len, int kv_len,
                                         fa_block_mask* out);

/* Quantize bf16 q, k, v for the quantized forward (the int8-QK / fp8-PV attention form of
 * FlashRT-Structures PR #1, "LTX-2.5 attention forms"). All tensors are [B, H, L, 128] on the
 * device, D contiguous; q, k, v are FA_BF16 with scale = NULL; q8 and k8 are FA_I8 and v8 is
 * FA_FP8_E4M3, with the shapes of their sources, data 16-byte aligned and strides multiples of
 * 16 elements. Outputs (caller-owned, written on `stream`):
 *   q8/k8 data: int8 codes; q8->scale / k8->scale: float32 [B][H][ceil(L/128)], one scale per
 *     128-token block: scale = amax / 127, code = round-half-even(x / scale) clamped to +-127
 *     (amax = 0 gives scale 0 and codes 0);
 *   v8 data: OCP E4M3 codes; v8->scale: float32 [B][H][128], one scale per channel over all
 *     tokens: scale = amax / 448, code = E4M3(x / scale) rounded half-even (scale 0: code 0).
 * The `scale` pointers of q8, k8 and v8 are written despite their const qualifier. */
fa_status flexattn_quantize_qkv(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                                fa_tensor* q8, fa_tensor* k8, fa_tensor* v8, hipStream_t stream);

/* Refinements of the quantized form (FlashRT-Structures PR #1, "LTX-2.5 attention forms": the
 * sage2 form scales Q/K per warp or per thread; the fused prep of its FP4 sibling centres the
 * inputs and applies a delta correction). As flexattn_quantize_qkv, plus:
 *   - qk_block: tokens per Q/K scale, 128 or 32 (32 = one wave of 32 queries, or one 32-key
 *     sub-block of the forward); q8->scale / k8->scale are float32 [B][H][ceil(L / qk_block)];
 *   - K centering when k_mean != NULL: mean[b][h][c] = (sum over tokens of K, exact while it fits
 *     a double) / L, rounded to float32, written to k_mean (float32 [B][Hkv][128]); K is quantized
 *     as K - mean (one float32 subtraction per element), which leaves softmax(q.k) unchanged and
 *     moves each score row by -(q . mean) * sm_scale; q_delta (float32 [B][Hq][Lq], required with
 *     k_mean unless B * Lq = 0) receives q_i . mean of the row's kv head, which
 *     flexattn_fwd_quant adds back to lse;
 *   - workspace: flexattn_quantize_qkv_ex_workspace_bytes(B, Hkv, Lkv) bytes, 16-byte aligned,
 *     used only with centering (fp64 partial sums of the mean; contents afterwards unspecified).
 * qk_block other than 128 or 32 is FA_ERR_UNSUPPORTED. */
size_t flexattn_quantize_qkv_ex_workspace_bytes(int B, int Hkv, int Lkv);
fa_status flexattn_quantize_qkv_ex(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, fa_tensor* q8,
                                   fa_tensor* k8, fa_tensor* v8, int qk_block, float* k_mean, float* q_delta,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Quantized forward for the output of flexattn_quantize_qkv_ex: q8, k8 FA_I8 and v8 FA_FP8_E4M3
 * with their scale arrays at qk_block tokens per Q/K scale (128 or 32, as quantized), out FA_BF16.
 * q_delta (may be NULL without centering) is the array flexattn_quantize_qkv_ex wrote: lse gets
 * sm_scale * q_delta[row] added, so it is the lse of the uncentred scores. Unmasked attention
 * without score_mod, as the quantized path of flexattn_fwd (which is this call with qk_block 128
 * and q_delta NULL). */
fa_status flexattn_fwd_quant(const fa_tensor* q8, const fa_tensor* k8, const fa_tensor* v8, int qk_block,
                             const float* q_delta, const fa_params* p, fa_tensor* out, float* lse, hipStream_t stream);

/* Device scratch of flexattn_fwd for the given operands: always 0. Every forward form (bf16, fp32,
 * quantized) keeps its scores, probabilities and running softmax state in registers and LDS
 * (FlexAttention guide, "Fused Triton JIT Kernel Compilation", item 3: intermediates stay on
 * chip), so flexattn_fwd takes no workspace argument. Kept so that a caller following the
 * caller-owned-workspace convention can size every call alike. */
size_t flexattn_fwd_workspace_bytes(const fa_tensor* q, const fa_tensor* k, int mask_kind, int score_kind);

/* Forward pass. q [B][Hq][Lq][D], k and v [B][Hkv][Lkv][D], out [B][Hq][Lq][D],
 * lse [B][Hq][Lq] float32 contiguous (natural log; may be NULL). Supported envelope:
 *   - D = 128;
 *   - dtypes: all FA_F32 (float32 MFMA, fp32 softmax); all FA_BF16 (bf16 MFMA with fp32
 *     accumulation and softmax; P rounded to bf16 before P.V); or the quantized form q, k FA_I8
 *     and v FA_FP8_E4M3 as written by flexattn_quantize_qkv (their scale arrays set) with out
 *     FA_BF16: Q.K^T on int8 MFMA, P coded as E4M3(448 P), P.V on fp8 MFMA. The quantized form
 *     serves unmasked attention only (mask_kind NONE, score_kind NONE, bm NULL; anything else is
 *     FA_ERR_UNSUPPORTED, as the page's attention form refuses masked sites);
 *   - Hq a multiple of Hkv (GQA: query head h reads kv head h / (Hq / Hkv));
 *   - data pointers 16-byte aligned and stride_b/h/l multiples of 8 elements (bf16) or
 *     4 elements (f32);
 *   - bm->q_block = 128, or 256 for bf16 (256-query workgroups), and bm->kv_block in {64, 128}.
 * `bm` may be NULL only when mask_kind is FA_MASK_NONE: every tile is then full (bf16 uses
 * 256-query workgroups when that still gives at least 256 of them).
 * The kernel trusts the BlockMask for which tiles to visit and evaluates mask_kind on partial
 * tiles (and on the ragged last kv block) only, like FlexAttention: a BlockMask built for a
 * different mask gives results for that mask's tile set.
 * A query row with no allowed key produces out = 0 and lse = -inf. */
fa_status flexattn_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                       const fa_block_mask* bm, int mask_kind, int score_kind, const fa_params* p,
                       fa_tensor* out, float* lse, hipStream_t stream);

/* Split-KV forward (the decoding form: few queries against many keys, FlexAttention wiki,
 * "flex_decoding"): the same result as flexattn_fwd, computed by cutting each work item's
 * (batch, query head, 128-query block) BlockMask tile list into n_splits contiguous ranges that
 * run as separate workgroups, so that a handful of query rows still fills the GPU. Each range
 * writes its normalised output and natural-log lse to `workspace`; a second kernel combines
 * them per row with weights exp(lse_s - lse), lse = log sum_s exp(lse_s).
 *   - bf16 only (FA_ERR_UNSUPPORTED otherwise, and for the quantized form or q_block 256);
 *   - n_splits in [1, 256] (1 is flexattn_fwd and needs no workspace);
 *   - workspace: device, 16-byte aligned, flexattn_fwd_splitkv_workspace_bytes(B, Hq, Lq,
 *     n_splits) bytes (fp32 partial outputs [n_splits][B][Hq][Lq][128], then their lse); its
 *     contents after the call are unspecified. Everything else as flexattn_fwd. */
size_t flexattn_fwd_splitkv_workspace_bytes(int B, int Hq, int Lq, int n_splits);
fa_status flexattn_fwd_splitkv(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_block_mask* bm,
                               int mask_kind, int score_kind, const fa_params* p, fa_tensor* out, float* lse,
                               int n_splits, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Column view of a BlockMask, for a backward that walks kv blocks (field names as in
 * FlexAttention's BlockMask; the pages give no layout). For each mask row (bm, hm) and kv block
 * kb, the q blocks whose (qb, kb) tile is partial (q_indices) or full (full_q_indices), each
 * list ascending with its length in the matching *_num_blocks entry and the unused tail 0.
 * Shapes (int32, device):
 *   q_num_blocks, full_q_num_blocks : [Bm][Hm][n_kvb]   (flexattn_block_mask_count_bytes(Bm, Hm,
 *                                                          kv_len, kv_block) bytes each)
 *   q_indices, full_q_indices       : [Bm][Hm][n_kvb][n_qb]  (flexattn_block_mask_index_bytes)
 * col_order (optional, int32 [Bm][Hm][n_kvb], NULL when unused) is the columns' schedule, as
 * row_order is the rows': the kv blocks of each row set by decreasing cost 4 * full + 5 * partial
 * live tiles, ties by increasing kv block (identity when n_kvb > 8192). The transpose fills it
 * when the pointer is set; the dk/dv pass of flexattn_bwd then starts the costliest columns
 * first. Results are identical with or without it. */
typedef struct {
  int32_t Bm, Hm, q_len, kv_len, q_block, kv_block, n_qb, n_kvb;
  int32_t* q_num_blocks;
  int32_t* q_indices;
  int32_t* full_q_num_blocks;
  int32_t* full_q_indices;
  int32_t* col_order;
} fa_block_mask_transposed;

/* Transpose a BlockMask into its column view on the device (the same tiles and classes, listed
 * per kv block). `out` carries the dimensions of `bm` (all eight must be equal) and four
 * caller-owned arrays; every entry of them is written. */
fa_status flexattn_block_mask_transpose(const fa_block_mask* bm, fa_block_mask_transposed* out, hipStream_t stream);

/* Device scratch of flexattn_bwd: per query row lse * log2(e) and delta = dout . out (float32
 * [B][Hq][Lq] each, padded to 16 bytes), then the slope-gradient partials (float32
 * [B][Hq][ceil(Lq / 128)]). */
size_t flexattn_bwd_workspace_bytes(int B, int Hq, int Lq);

/* Backward pass of flexattn_fwd (FlexAttention guide, "Systems Mechanics", item 2: the backward
 * gives dQ, dK, dV, differentiates the score_mod, and passes gradients to learnable score_mod
 * parameters such as ALiBi slopes). With f the modified score of an allowed pair and
 * P = exp(f - lse):
 *   dv = P^T dout;  dA = P (dout v^T - rowsum(dout * out)) * (1 - (f / softcap)^2 under SOFTCAP);
 *   dq = sm_scale dA k;  dk = sm_scale dA^T q;  dslopes[h] = -sum over (b, i, j) of dA |i - j|.
 * GQA: dk and dv of a kv head sum over its query heads.
 *   - all tensors FA_BF16 with D = 128: q, out, dout, dq [B][Hq][Lq]; k, v, dk, dv [B][Hkv][Lkv];
 *     element strides as in flexattn_fwd; gradients written in bf16 (fp32 accumulation);
 *   - out and lse are those of flexattn_fwd on the same inputs (lse natural log, float32
 *     [B][Hq][Lq] contiguous; -inf rows get zero gradients);
 *   - bm and bmt: the forward's BlockMask and its transpose (flexattn_block_mask_transpose), both
 *     with 128 x 128 tiles and Hm = 1 (otherwise FA_ERR_UNSUPPORTED), or both NULL with mask_kind
 *     NONE. As in the forward the BlockMask decides which tiles are visited and mask_kind is
 *     evaluated on partial tiles;
 *   - dslopes: float32 [Hq] device, overwritten with the slope gradient summed over batches; NULL
 *     skips it; only allowed with ALIBI;
 *   - workspace: flexattn_bwd_workspace_bytes(B, Hq, Lq) bytes, 16-byte aligned; contents after
 *     the call unspecified.
 * dq, dk and dv are overwritten (not accumulated into). Everything else as flexattn_fwd. */
fa_status flexattn_bwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                       const fa_tensor* dout, const float* lse, const fa_block_mask* bm,
                       const fa_block_mask_transposed* bmt, int mask_kind, int score_kind, const fa_params* p,
                       fa_tensor* dq, fa_tensor* dk, fa_tensor* dv, float* dslopes, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char* flexattn_last_error(void);

/* ABI version (major * 100 + minor). */
int flexattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLEXATTN_H */

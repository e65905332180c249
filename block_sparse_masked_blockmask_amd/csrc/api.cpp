// C-ABI layer: argument validation, error reporting and kernel selection. Every check happens
// on the host before anything is enqueued, so a non-OK status never leaves partial writes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include <vector>

#include "api_internal.h"
#include "flexattn.h"
#include "launch.h"
#include "tile_class.h"

namespace fa_api {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa_status ok() {
  g_last_error.clear();
  return FA_OK;
}

int cdiv(int a, int b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const int kValidMask = FA_MASK_DOC | FA_MASK_CAUSAL | FA_MASK_WINDOW | FA_MASK_PREFIX_LM;
const int kValidScore = FA_SCORE_ALIBI | FA_SCORE_SOFTCAP;

// The kernels are built for gfx950 only. Every launching entry point checks, after validating
// its arguments and before enqueuing anything, that the current device is a gfx950; another
// device is refused with FA_ERR_UNSUPPORTED and its architecture name. The name is read once
// per device and cached. FLEXATTN_DEVICE_ARCH, when set, replaces the device's name (a test
// hook: it lets the refusal be checked on a machine without that device).
std::mutex g_arch_mu;
std::string g_arch_name[kMaxDevices];

bool arch_is_gfx950(const std::string& name) {
  // hipDeviceProp_t::gcnArchName is "gfx950" followed by optional ":feature+/-" suffixes.
  return name.compare(0, 6, "gfx950") == 0 && (name.size() == 6 || name[6] == ':');
}

fa_status check_device() {
  std::string name;
  const char* over = std::getenv("FLEXATTN_DEVICE_ARCH");
  if (over != nullptr && *over != '\0') {
    name = over;
  } else {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FA_ERR_DEVICE, "no current HIP device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_arch_mu);
    if (g_arch_name[dev].empty()) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return fail(FA_ERR_DEVICE, "cannot read device %d properties: %s", dev, hipGetErrorString(e));
      g_arch_name[dev] = prop.gcnArchName[0] ? prop.gcnArchName : "unknown";
    }
    name = g_arch_name[dev];
  }
  if (!arch_is_gfx950(name))
    return fail(FA_ERR_UNSUPPORTED, "device %s is not gfx950: the kernels are built for gfx950 only", name.c_str());
  return FA_OK;
}

// FLEXATTN_VERIFY_BLOCKMASK (debug): when set to a non-empty value other than "0", the forward
// and the backward copy the BlockMask lists they are given to the host, synchronising the
// stream, and check them before enqueuing anything: every count in [0, n], every listed block in
// [0, n) and strictly ascending, no block both full and partial in one row. A violation is
// FA_ERR_INVALID_ARG naming the row. The kernels themselves clamp counts and skip entries out of
// range (so that a corrupt BlockMask cannot send them outside its arrays), which hides such
// errors; this mode shows them. It synchronises the host, so it is not for graph capture.
bool verify_enabled() {
  const char* v = std::getenv("FLEXATTN_VERIFY_BLOCKMASK");
  return v != nullptr && *v != '\0' && std::strcmp(v, "0") != 0;
}

// rows lists of up to n entries (full and partial), counts [rows], indices [rows][n].
fa_status verify_lists(const int32_t* full_num, const int32_t* full_idx, const int32_t* part_num,
                       const int32_t* part_idx, int64_t rows, int n, const char* what, hipStream_t stream) {
  if (rows <= 0 || n <= 0) return FA_OK;
  std::vector<int32_t> fn(rows), pn(rows), fi((size_t)rows * n), pi((size_t)rows * n);
  hipError_t e = hipSuccess;
  const size_t cb = (size_t)rows * sizeof(int32_t), ib = (size_t)rows * n * sizeof(int32_t);
  if (e == hipSuccess) e = hipMemcpyAsync(fn.data(), full_num, cb, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(pn.data(), part_num, cb, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(fi.data(), full_idx, ib, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(pi.data(), part_idx, ib, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(FA_ERR_DEVICE, "%s verification copy failed: %s", what, hipGetErrorString(e));
  std::vector<unsigned char> seen(n);
  for (int64_t r = 0; r < rows; ++r) {
    if (fn[r] < 0 || fn[r] > n || pn[r] < 0 || pn[r] > n)
      return fail(FA_ERR_INVALID_ARG, "%s row %lld: counts %d full, %d partial outside [0, %d]", what, (long long)r,
                  fn[r], pn[r], n);
    std::fill(seen.begin(), seen.end(), 0);
    for (int list = 0; list < 2; ++list) {
      const int32_t* idx = (list ? pi.data() : fi.data()) + (size_t)r * n;
      const int cnt = list ? pn[r] : fn[r];
      for (int i = 0; i < cnt; ++i) {
        if (idx[i] < 0 || idx[i] >= n)
          return fail(FA_ERR_INVALID_ARG, "%s row %lld: %s entry %d is %d, outside [0, %d)", what, (long long)r,
                      list ? "partial" : "full", i, idx[i], n);
        if (i > 0 && idx[i] <= idx[i - 1])
          return fail(FA_ERR_INVALID_ARG, "%s row %lld: %s list not strictly ascending at entry %d", what,
                      (long long)r, list ? "partial" : "full", i);
        if (seen[idx[i]])
          return fail(FA_ERR_INVALID_ARG, "%s row %lld: block %d is listed both full and partial", what,
                      (long long)r, idx[i]);
        seen[idx[i]] = 1;
      }
    }
  }
  return FA_OK;
}

// Checks shared by the builder and the forward pass for the mask parameters.
fa_status check_mask(int mask_kind, const fa_params* p, int Lq, int Lkv) {
  if (mask_kind & ~kValidMask) return fail(FA_ERR_INVALID_ARG, "unknown mask_kind bits 0x%x", mask_kind);
  if ((mask_kind & FA_MASK_PREFIX_LM) && (mask_kind & FA_MASK_CAUSAL))
    return fail(FA_ERR_INVALID_ARG, "PREFIX_LM already contains causal; do not combine it with CAUSAL");
  if (mask_kind != FA_MASK_NONE && p == nullptr) return fail(FA_ERR_INVALID_ARG, "params is NULL");
  if ((mask_kind & FA_MASK_WINDOW) && p->window <= 0) return fail(FA_ERR_INVALID_ARG, "window must be > 0");
  if ((mask_kind & FA_MASK_PREFIX_LM) && p->prefix_len < 0) return fail(FA_ERR_INVALID_ARG, "prefix_len must be >= 0");
  if ((mask_kind & FA_MASK_DOC) && ((Lq > 0 && p->q_doc == nullptr) || (Lkv > 0 && p->kv_doc == nullptr)))
    return fail(FA_ERR_INVALID_ARG, "DOC mask needs q_doc and kv_doc");
  return FA_OK;
}

// Checks of a BlockMask build request shared by the device and host builders.
fa_status check_build(int mask_kind, const fa_params* p, int B, int q_len, int kv_len, const fa_block_mask* out) {
  fa_status st = check_mask(mask_kind, p, q_len, kv_len);
  if (st != FA_OK) return st;
  if (out == nullptr) return fail(FA_ERR_INVALID_ARG, "out is NULL");
  if (B <= 0 || B > 65535) return fail(FA_ERR_INVALID_ARG, "B must be in [1, 65535] (got %d)", B);
  if (q_len < 0 || kv_len < 0) return fail(FA_ERR_INVALID_ARG, "negative sequence length");
  if (out->q_len != q_len || out->kv_len != kv_len)
    return fail(FA_ERR_INVALID_ARG, "out->q_len/kv_len (%d, %d) differ from q_len/kv_len (%d, %d)",
                out->q_len, out->kv_len, q_len, kv_len);
  if ((out->q_block != 64 && out->q_block != 128 && out->q_block != 256) ||
      (out->kv_block != 64 && out->kv_block != 128))
    return fail(FA_ERR_UNSUPPORTED, "block sizes must be q 64/128/256 and kv 64/128 (got %d x %d)", out->q_block,
                out->kv_block);
  if (out->n_qb != cdiv(q_len, out->q_block) || out->n_kvb != cdiv(kv_len, out->kv_block))
    return fail(FA_ERR_INVALID_ARG, "n_qb/n_kvb (%d, %d) do not match ceil(len / block)", out->n_qb, out->n_kvb);
  if (out->Hm != 1) return fail(FA_ERR_INVALID_ARG, "Hm must be 1: no mask flag depends on the head");
  if ((mask_kind & FA_MASK_DOC) ? out->Bm != B : (out->Bm != 1 && out->Bm != B))
    return fail(FA_ERR_INVALID_ARG, "Bm must be B with DOC, else 1 or B (got %d)", out->Bm);
  if (out->n_qb > 0 && (!out->kv_num_blocks || !out->full_kv_num_blocks))
    return fail(FA_ERR_INVALID_ARG, "BlockMask count arrays are NULL");
  if (out->n_qb > 0 && out->n_kvb > 0 && (!out->kv_indices || !out->full_kv_indices))
    return fail(FA_ERR_INVALID_ARG, "BlockMask index arrays are NULL");
  for (const void* ptr : {(const void*)out->kv_num_blocks, (const void*)out->full_kv_num_blocks,
                          (const void*)out->kv_indices, (const void*)out->full_kv_indices,
                          (const void*)out->row_order})
    if (reinterpret_cast<uintptr_t>(ptr) & 3u) return fail(FA_ERR_INVALID_ARG, "BlockMask arrays must be 4-byte aligned");
  return FA_OK;
}

}  // namespace fa_api

using namespace fa_api;

extern "C" {

const char* flexattn_last_error(void) { return g_last_error.c_str(); }

int flexattn_version(void) { return 100; }

size_t flexattn_block_mask_index_bytes(int Bm, int Hm, int q_len, int kv_len, int q_block, int kv_block) {
  if (Bm <= 0 || Hm <= 0 || q_len < 0 || kv_len < 0 || q_block <= 0 || kv_block <= 0) return 0;
  return (size_t)Bm * Hm * cdiv(q_len, q_block) * cdiv(kv_len, kv_block) * sizeof(int32_t);
}

size_t flexattn_block_mask_count_bytes(int Bm, int Hm, int q_len, int q_block) {
  if (Bm <= 0 || Hm <= 0 || q_len < 0 || q_block <= 0) return 0;
  return (size_t)Bm * Hm * cdiv(q_len, q_block) * sizeof(int32_t);
}

size_t flexattn_block_mask_bytes(int Bm, int Hm, int q_len, int kv_len, int q_block, int kv_block) {
  if (Bm <= 0 || Hm <= 0 || q_len < 0 || kv_len < 0 || q_block <= 0 || kv_block <= 0) return 0;
  return 2 * flexattn_block_mask_index_bytes(Bm, Hm, q_len, kv_len, q_block, kv_block) +
         2 * flexattn_block_mask_count_bytes(Bm, Hm, q_len, q_block);
}

size_t flexattn_block_mask_workspace_bytes(int mask_kind, int B, int q_len, int kv_len, int q_block, int kv_block) {
  if (!(mask_kind & FA_MASK_DOC) || B <= 0 || q_len < 0 || kv_len < 0 || q_block <= 0 || kv_block <= 0) return 0;
  return (size_t)B * (cdiv(q_len, q_block) + cdiv(kv_len, kv_block)) * 4 * sizeof(int32_t);
}

}  // extern "C"

namespace fa_api {

// Enqueue the device builder; `workspace` holds the per-block summaries (validated by the caller).
fa_status launch_build(int mask_kind, const fa_params* p, int B, int q_len, int kv_len, fa_block_mask* out,
                       void* workspace, size_t need, hipStream_t stream) {
  fa::BlockMaskArgs a{};
  a.flags = mask_kind;
  a.window = (mask_kind & FA_MASK_WINDOW) ? p->window : 0;
  a.prefix_len = (mask_kind & FA_MASK_PREFIX_LM) ? p->prefix_len : 0;
  a.B = B;
  a.Lq = q_len;
  a.Lkv = kv_len;
  a.BQ = out->q_block;
  a.BK = out->kv_block;
  a.nqb = out->n_qb;
  a.nkvb = out->n_kvb;
  a.Bm = out->Bm;
  a.q_doc = (mask_kind & FA_MASK_DOC) ? p->q_doc : nullptr;
  a.kv_doc = (mask_kind & FA_MASK_DOC) ? p->kv_doc : nullptr;
  if (need > 0) {
    a.qsum = static_cast<int*>(workspace);
    a.kvsum = a.qsum + (size_t)B * a.nqb * 4;
  }
  a.kv_num = out->kv_num_blocks;
  a.kv_idx = out->kv_indices;
  a.full_num = out->full_kv_num_blocks;
  a.full_idx = out->full_kv_indices;
  a.row_order = out->row_order;
  a.self_ids = (mask_kind & FA_MASK_DOC) && p->q_doc == p->kv_doc && q_len == kv_len;
  hipError_t e = fa::launch_block_mask(a, stream);
  if (e != hipSuccess) return fail(FA_ERR_DEVICE, "block mask launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace fa_api

extern "C" {

fa_status flexattn_block_mask_build(int mask_kind, const fa_params* p, int B, int q_len, int kv_len,
                                    fa_block_mask* out, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  fa_status st = check_build(mask_kind, p, B, q_len, kv_len, out);
  if (st != FA_OK) return st;
  const size_t need = flexattn_block_mask_workspace_bytes(mask_kind, B, q_len, kv_len, out->q_block, out->kv_block);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(FA_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (need > 0 && !aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if ((st = check_device()) != FA_OK) return st;
  return launch_build(mask_kind, p, B, q_len, kv_len, out, workspace, need, stream);
}


fa_status flexattn_block_mask_build_host(int mask_kind, const fa_params* p, int B, int q_len, int kv_len,
                                         fa_block_mask* out) {
  fa_status st = check_build(mask_kind, p, B, q_len, kv_len, out);
  if (st != FA_OK) return st;
  const int flags = mask_kind;
  const int window = (mask_kind & FA_MASK_WINDOW) ? p->window : 0;
  const int prefix_len = (mask_kind & FA_MASK_PREFIX_LM) ? p->prefix_len : 0;
  const bool doc = (mask_kind & FA_MASK_DOC) != 0;
  const int BQ = out->q_block, BK = out->kv_block, nqb = out->n_qb, nkvb = out->n_kvb;
  const bool self_ids = doc && p->q_doc == p->kv_doc && q_len == kv_len;
  // Per-block document-id summaries of one batch: [min, max, dense] (see tile_class.h).
  auto summarise = [](const int32_t* ids, int L, int blk, int n, std::vector<int>& sum) {
    sum.assign((size_t)3 * n, 0);
    for (int x = 0; x < n; ++x) {
      const int lo = x * blk, hi = std::min(L, lo + blk);
      int mn = ids[lo], mx = ids[lo], dense = 1;
      for (int i = lo + 1; i < hi; ++i) {
        mn = std::min(mn, ids[i]);
        mx = std::max(mx, ids[i]);
        const int inc = ids[i] - ids[i - 1];
        if (inc != 0 && inc != 1) dense = 0;
      }
      sum[3 * x] = mn;
      sum[3 * x + 1] = mx;
      sum[3 * x + 2] = dense;
    }
  };
  std::vector<int> qs, ks;
  for (int bm = 0; bm < out->Bm; ++bm) {
    const int b = out->Bm == B ? bm : 0;  // without DOC no predicate depends on the batch
    const int32_t* qd = doc ? p->q_doc + (size_t)b * q_len : nullptr;
    const int32_t* kd = doc ? p->kv_doc + (size_t)b * kv_len : nullptr;
    if (doc) {
      summarise(qd, q_len, BQ, nqb, qs);
      summarise(kd, kv_len, BK, nkvb, ks);
    }
    for (int qb = 0; qb < nqb; ++qb) {
      const size_t row = (size_t)bm * nqb + qb;  // Hm = 1
      int32_t* full = out->full_kv_indices + row * nkvb;
      int32_t* part = out->kv_indices + row * nkvb;
      const int q0 = qb * BQ, q1 = std::min(q_len, q0 + BQ);
      int nf = 0, np = 0;
      for (int kb = 0; kb < nkvb; ++kb) {
        const int k0 = kb * BK, k1 = std::min(kv_len, k0 + BK);
        int cls = fa::classify_closed(flags, window, prefix_len, q0, q1, k0, k1, doc ? qs[3 * qb] : 0,
                                      doc ? qs[3 * qb + 1] : 0, doc ? qs[3 * qb + 2] : 0, doc ? ks[3 * kb] : 0,
                                      doc ? ks[3 * kb + 1] : 0, doc ? ks[3 * kb + 2] : 0,
                                      self_ids);
        if (cls == 3) {  // every in-range pair, until one is allowed
          cls = 0;
          for (int i = q0; i < q1 && !cls; ++i)
            for (int j = k0; j < k1; ++j)
              if (fa::mask_pair_flags(flags, window, prefix_len, i, j, doc ? qd[i] : 0, doc ? kd[j] : 0)) {
                cls = 1;
                break;
              }
        }
        if (cls == 2) full[nf++] = kb;
        if (cls == 1) part[np++] = kb;
      }
      for (int j = nf; j < nkvb; ++j) full[j] = 0;
      for (int j = np; j < nkvb; ++j) part[j] = 0;
      out->full_kv_num_blocks[row] = nf;
      out->kv_num_blocks[row] = np;
    }
    if (out->row_order) {
      int32_t* order = out->row_order + (size_t)bm * nqb;
      if (nqb > fa::kRowOrderMax) {
        for (int qb = 0; qb < nqb; ++qb) order[qb] = qb;
      } else {
        std::vector<uint32_t> keys(nqb);
        for (int qb = 0; qb < nqb; ++qb) {
          const size_t row = (size_t)bm * nqb + qb;
          keys[qb] = fa::row_order_key(out->full_kv_num_blocks[row], out->kv_num_blocks[row], qb);
        }
        std::sort(keys.begin(), keys.end());
        for (int r = 0; r < nqb; ++r) order[r] = (int32_t)(keys[r] & fa::kRowOrderQbMask);
      }
    }
  }
  return ok();
}

static fa_status check_tensor(const fa_tensor* t, const char* name, int elem_align) {
  if (t == nullptr) return fail(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if (t->B < 0 || t->H <= 0 || t->L < 0 || t->D <= 0) return fail(FA_ERR_INVALID_ARG, "%s has invalid shape", name);
  if (t->data == nullptr && (int64_t)t->B * t->L > 0) return fail(FA_ERR_INVALID_ARG, "%s->data is NULL", name);
  if (!aligned16(t->data)) return fail(FA_ERR_INVALID_ARG, "%s->data must be 16-byte aligned", name);
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_l < t->D)
    return fail(FA_ERR_INVALID_ARG, "%s strides must be non-negative with stride_l >= D", name);
  if (t->stride_l > (1 << 24)) return fail(FA_ERR_UNSUPPORTED, "%s->stride_l above 2^24 elements", name);
  if (t->stride_b % elem_align || t->stride_h % elem_align || t->stride_l % elem_align)
    return fail(FA_ERR_INVALID_ARG, "%s strides must be multiples of %d elements", name, elem_align);
  if (t->scale != nullptr) return fail(FA_ERR_INVALID_ARG, "%s->scale must be NULL for this dtype", name);
  return FA_OK;
}

static fa_status fwd_quantized(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_block_mask* bm,
                               int mask_kind, int score_kind, const fa_params* p, fa_tensor* out, float* lse,
                               int qk_block, const float* q_delta, hipStream_t stream);

size_t flexattn_fwd_workspace_bytes(const fa_tensor* q, const fa_tensor* k, int mask_kind, int score_kind) {
  (void)q;
  (void)k;
  (void)mask_kind;
  (void)score_kind;
  return 0;  // every forward form keeps its intermediates in registers and LDS
}

size_t flexattn_fwd_splitkv_workspace_bytes(int B, int Hq, int Lq, int n_splits) {
  if (B < 0 || Hq < 0 || Lq < 0 || n_splits < 1) return 0;
  return (size_t)n_splits * B * Hq * Lq * (128 + 1) * sizeof(float);
}

}  // extern "C"

namespace {

// The forward with nsplit contiguous ranges of each work item's tile list (nsplit = 1: the
// plain forward; nsplit > 1: partial results in the workspace, then the merge).
fa_status fwd_impl(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_block_mask* bm,
                   int mask_kind, int score_kind, const fa_params* p, fa_tensor* out, float* lse, int nsplit,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int dt = q->dtype;
  if (k->dtype != dt || v->dtype != dt || out->dtype != dt)
    return fail(FA_ERR_INVALID_ARG, "q, k, v and out must share one dtype");
  if (dt != FA_F32 && dt != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not served by flexattn_fwd (f32 or bf16)", dt);
  const int ea = dt == FA_BF16 ? 8 : 4;
  fa_status st;
  if ((st = check_tensor(q, "q", ea)) != FA_OK) return st;
  if ((st = check_tensor(k, "k", ea)) != FA_OK) return st;
  if ((st = check_tensor(v, "v", ea)) != FA_OK) return st;
  if ((st = check_tensor(out, "out", ea)) != FA_OK) return st;
  if (q->D != 128 || k->D != 128 || v->D != 128 || out->D != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dim must be 128 (got q %d, k %d, v %d)", q->D, k->D, v->D);
  if (k->B != q->B || v->B != q->B || out->B != q->B) return fail(FA_ERR_INVALID_ARG, "batch sizes differ");
  if (k->H != v->H || k->L != v->L) return fail(FA_ERR_INVALID_ARG, "k and v shapes differ");
  if (q->H % k->H != 0) return fail(FA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", q->H, k->H);
  if (out->H != q->H || out->L != q->L) return fail(FA_ERR_INVALID_ARG, "out shape differs from q");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if ((st = check_mask(mask_kind, p, q->L, k->L)) != FA_OK) return st;
  if (score_kind & ~kValidScore) return fail(FA_ERR_INVALID_ARG, "unknown score_kind bits 0x%x", score_kind);
  if (score_kind != FA_SCORE_NONE && p == nullptr) return fail(FA_ERR_INVALID_ARG, "params is NULL");
  if ((score_kind & FA_SCORE_ALIBI) && p->alibi_slopes == nullptr)
    return fail(FA_ERR_INVALID_ARG, "ALIBI needs alibi_slopes");
  if ((score_kind & FA_SCORE_SOFTCAP) && !(p->softcap > 0.f) )
    return fail(FA_ERR_INVALID_ARG, "SOFTCAP needs softcap > 0");

  const int B = q->B, Lq = q->L, Lkv = k->L;
  int kv_block = 128, q_block = 128;
  bool dense = false;
  fa::FwdArgs a{};
  if (bm == nullptr) {
    if (mask_kind != FA_MASK_NONE) return fail(FA_ERR_INVALID_ARG, "a BlockMask is required unless mask_kind is NONE");
    // bf16 without a BlockMask runs the software-pipelined every-tile-full kernel (256-query
    // workgroups).
    dense = dt == FA_BF16 && nsplit == 1;
    if (dense) q_block = 256;
    a.all_full = 1;
    a.Bm = a.Hm = 1;
    a.nqb = cdiv(Lq, q_block);
    a.nkvb = cdiv(Lkv, kv_block);
  } else {
    if (bm->q_len != Lq || bm->kv_len != Lkv)
      return fail(FA_ERR_INVALID_ARG, "BlockMask was built for lengths (%d, %d), not (%d, %d)", bm->q_len, bm->kv_len, Lq, Lkv);
    if (bm->q_block != 128 && !(dt == FA_BF16 && bm->q_block == 256))
      return fail(FA_ERR_UNSUPPORTED, "q_block must be 128 (or 256 for bf16) (got %d)", bm->q_block);
    q_block = bm->q_block;
    if (bm->kv_block != 64 && bm->kv_block != 128)
      return fail(FA_ERR_UNSUPPORTED, "kv_block must be 64 or 128 (got %d)", bm->kv_block);
    if (bm->n_qb != cdiv(Lq, bm->q_block) || bm->n_kvb != cdiv(Lkv, bm->kv_block))
      return fail(FA_ERR_INVALID_ARG, "BlockMask n_qb/n_kvb do not match its lengths and block sizes");
    if (bm->Bm != 1 && bm->Bm != B) return fail(FA_ERR_INVALID_ARG, "BlockMask Bm must be 1 or B");
    if (bm->Hm != 1 && bm->Hm != q->H) return fail(FA_ERR_INVALID_ARG, "BlockMask Hm must be 1 or Hq");
    if (bm->n_qb > 0 && (!bm->kv_num_blocks || !bm->full_kv_num_blocks || (bm->n_kvb > 0 && (!bm->kv_indices || !bm->full_kv_indices))))
      return fail(FA_ERR_INVALID_ARG, "BlockMask arrays are NULL");
    kv_block = bm->kv_block;
    a.all_full = 0;
    a.Bm = bm->Bm;
    a.Hm = bm->Hm;
    a.row_order = nsplit == 1 && bm->n_qb > 0 ? bm->row_order : nullptr;  // schedule only
    a.nqb = bm->n_qb;
    a.nkvb = bm->n_kvb;
    a.kv_num = bm->kv_num_blocks;
    a.kv_idx = bm->kv_indices;
    a.full_num = bm->full_kv_num_blocks;
    a.full_idx = bm->full_kv_indices;
    if (verify_enabled()) {
      st = verify_lists(bm->full_kv_num_blocks, bm->full_kv_indices, bm->kv_num_blocks, bm->kv_indices,
                        (int64_t)bm->Bm * bm->Hm * bm->n_qb, bm->n_kvb, "BlockMask", stream);
      if (st != FA_OK) return st;
    }
  }
  if (nsplit > 1) {
    if (dt != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "split-KV serves bf16 tensors");
    if (q_block != 128) return fail(FA_ERR_UNSUPPORTED, "split-KV needs q_block 128 (got %d)", q_block);
    const size_t need = flexattn_fwd_splitkv_workspace_bytes(B, q->H, Lq, nsplit);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
      return fail(FA_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    if (need > 0 && !aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  // Split-KV with grouped query heads: when all queries of all heads of a kv group fit one
  // 128-row workgroup (and the BlockMask does not depend on the head), one workgroup per kv head
  // computes them all and each K/V tile is read once for the group.
  const int group = q->H / k->H;
  a.pack = (nsplit > 1 && group > 1 && (int64_t)group * Lq <= 128 && (bm == nullptr || bm->Hm == 1)) ? 1 : 0;
  const int64_t total = (int64_t)B * (a.pack ? k->H : q->H) * a.nqb * nsplit;
  if (total > 0x7fffffff) return fail(FA_ERR_UNSUPPORTED, "grid too large (%lld workgroups)", (long long)total);

  a.q = q->data; a.k = k->data; a.v = v->data; a.o = out->data; a.lse = lse;
  a.q_sb = q->stride_b; a.q_sh = q->stride_h; a.q_sl = q->stride_l;
  a.k_sb = k->stride_b; a.k_sh = k->stride_h; a.k_sl = k->stride_l;
  a.v_sb = v->stride_b; a.v_sh = v->stride_h; a.v_sl = v->stride_l;
  a.o_sb = out->stride_b; a.o_sh = out->stride_h; a.o_sl = out->stride_l;
  a.B = B; a.Hq = q->H; a.Hkv = k->H; a.Lq = Lq; a.Lkv = Lkv; a.group = q->H / k->H;
  a.flags = mask_kind;
  a.window = (mask_kind & FA_MASK_WINDOW) ? p->window : 0;
  a.prefix_len = (mask_kind & FA_MASK_PREFIX_LM) ? p->prefix_len : 0;
  a.q_doc = (mask_kind & FA_MASK_DOC) ? p->q_doc : nullptr;
  a.kv_doc = (mask_kind & FA_MASK_DOC) ? p->kv_doc : nullptr;
  const float sm = (p && p->sm_scale > 0.f) ? p->sm_scale : 1.0f / std::sqrt((float)q->D);
  a.sm_scale = sm;
  a.scale_log2 = sm * 1.4426950408889634f;
  a.softcap = (score_kind & FA_SCORE_SOFTCAP) ? p->softcap : 0.f;
  a.inv_softcap = (score_kind & FA_SCORE_SOFTCAP) ? 1.0f / p->softcap : 0.f;
  {
    // score_mod constants folded into the log2 domain (see score_log2 in fwd.hip).
    const double l2e = 1.4426950408889634;
    const double cap = (score_kind & FA_SCORE_SOFTCAP) ? (double)p->softcap : 1.0;
    a.sc_in = (float)((double)sm * 2.0 * l2e / cap);
    a.sc_out = (float)(cap * l2e);
    a.sc_out2 = (float)(-2.0 * cap * l2e);
    a.slope_mul = (float)((score_kind & FA_SCORE_SOFTCAP) ? 2.0 * l2e / cap : l2e);
  }
  a.slopes = (score_kind & FA_SCORE_ALIBI) ? p->alibi_slopes : nullptr;
  a.total_wg = (int)total;
  a.nsplit = nsplit;
  if ((st = check_device()) != FA_OK) return st;
  if (nsplit > 1) {
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = a.part_o + (size_t)nsplit * B * q->H * Lq * 128;
  }
  // bf16 with a BlockMask of 128-query blocks and a mask without document ids (one key interval
  // per query) runs the software-pipelined block-sparse kernel; document masks, 256-query blocks,
  // split-KV and fp32 run the kernels of fwd.hip.
  const bool pipe = !dense && dt == FA_BF16 && nsplit == 1 && bm != nullptr && q_block == 128 &&
                    !(mask_kind & FA_MASK_DOC);
  hipError_t e = dense ? fa::launch_fwd_dense(a, score_kind, stream)
                 : pipe ? fa::launch_fwd_pipe(a, kv_block, score_kind, stream)
                        : fa::launch_fwd(a, dt == FA_BF16 ? 1 : 0, q_block, kv_block, score_kind, stream);
  if (e != hipSuccess) return fail(FA_ERR_DEVICE, "forward launch failed: %s", hipGetErrorString(e));
  if (nsplit > 1) {
    fa::MergeArgs m{};
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.o = static_cast<__bf16*>(out->data);
    m.lse = lse;
    m.o_sb = out->stride_b;
    m.o_sh = out->stride_h;
    m.o_sl = out->stride_l;
    m.B = B;
    m.Hq = q->H;
    m.Lq = Lq;
    m.nsplit = nsplit;
    e = fa::launch_splitkv_merge(m, stream);
    if (e != hipSuccess) return fail(FA_ERR_DEVICE, "split-KV merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

fa_status flexattn_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_block_mask* bm,
                       int mask_kind, int score_kind, const fa_params* p, fa_tensor* out, float* lse,
                       hipStream_t stream) {
  if (!q || !k || !v || !out) return fail(FA_ERR_INVALID_ARG, "q, k, v and out must not be NULL");
  if (q->dtype == FA_I8) return fwd_quantized(q, k, v, bm, mask_kind, score_kind, p, out, lse, 128, nullptr, stream);
  return fwd_impl(q, k, v, bm, mask_kind, score_kind, p, out, lse, 1, nullptr, 0, stream);
}

fa_status flexattn_fwd_splitkv(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_block_mask* bm,
                               int mask_kind, int score_kind, const fa_params* p, fa_tensor* out, float* lse,
                               int n_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out) return fail(FA_ERR_INVALID_ARG, "q, k, v and out must not be NULL");
  if (n_splits < 1 || n_splits > 256) return fail(FA_ERR_INVALID_ARG, "n_splits must be in [1, 256] (got %d)", n_splits);
  if (q->dtype == FA_I8) return fail(FA_ERR_UNSUPPORTED, "split-KV does not serve the quantized form");
  return fwd_impl(q, k, v, bm, mask_kind, score_kind, p, out, lse, n_splits, workspace, workspace_bytes, stream);
}

fa_status flexattn_fwd_quant(const fa_tensor* q8, const fa_tensor* k8, const fa_tensor* v8, int qk_block,
                             const float* q_delta, const fa_params* p, fa_tensor* out, float* lse, hipStream_t stream) {
  if (!q8 || !k8 || !v8 || !out) return fail(FA_ERR_INVALID_ARG, "q8, k8, v8 and out must not be NULL");
  return fwd_quantized(q8, k8, v8, nullptr, FA_MASK_NONE, FA_SCORE_NONE, p, out, lse, qk_block, q_delta, stream);
}

// A quantized tensor's scale array may be NULL only where it has no entries: Q and K scales are
// per block of rows (none without rows), V scales per channel (always some while B > 0).
static bool needs_scale(const fa_tensor* t, int rows) { return t->scale == nullptr && (int64_t)t->B * rows > 0; }

static fa_status check_q_tensor(const fa_tensor* t, const char* name, int dtype, int elem_align) {
  if (t == nullptr) return fail(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if (t->dtype != dtype) return fail(FA_ERR_INVALID_ARG, "%s has dtype %d, expected %d", name, t->dtype, dtype);
  if (t->B < 0 || t->H <= 0 || t->L < 0 || t->D != 128)
    return fail(t->D != 128 ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG, "%s must be [B, H, L, 128]", name);
  if (t->data == nullptr && (int64_t)t->B * t->L > 0) return fail(FA_ERR_INVALID_ARG, "%s->data is NULL", name);
  if (!aligned16(t->data)) return fail(FA_ERR_INVALID_ARG, "%s->data must be 16-byte aligned", name);
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_l < t->D || t->stride_l > (1 << 24))
    return fail(FA_ERR_INVALID_ARG, "%s has invalid strides", name);
  if (t->stride_b % elem_align || t->stride_h % elem_align || t->stride_l % elem_align)
    return fail(FA_ERR_INVALID_ARG, "%s strides must be multiples of %d elements", name, elem_align);
  return FA_OK;
}

size_t flexattn_quantize_qkv_ex_workspace_bytes(int B, int Hkv, int Lkv) {
  if (B < 0 || Hkv < 0 || Lkv < 0) return 0;
  return (size_t)B * Hkv * fa::quant_mean_chunks(Lkv) * 128 * sizeof(double);
}

static fa_status quantize_impl(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, fa_tensor* q8,
                               fa_tensor* k8, fa_tensor* v8, int qk_block, float* k_mean, float* q_delta,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa_status st;
  if (qk_block != 128 && qk_block != 32) return fail(FA_ERR_UNSUPPORTED, "qk_block must be 128 or 32 (got %d)", qk_block);
  if ((st = check_q_tensor(q, "q", FA_BF16, 8)) != FA_OK) return st;
  if ((st = check_q_tensor(k, "k", FA_BF16, 8)) != FA_OK) return st;
  if ((st = check_q_tensor(v, "v", FA_BF16, 8)) != FA_OK) return st;
  if ((st = check_q_tensor(q8, "q8", FA_I8, 16)) != FA_OK) return st;
  if ((st = check_q_tensor(k8, "k8", FA_I8, 16)) != FA_OK) return st;
  if ((st = check_q_tensor(v8, "v8", FA_FP8_E4M3, 16)) != FA_OK) return st;
  if (q->scale || k->scale || v->scale) return fail(FA_ERR_INVALID_ARG, "bf16 sources carry no scale");
  if (needs_scale(q8, q8->L) || needs_scale(k8, k8->L) || needs_scale(v8, 1))
    return fail(FA_ERR_INVALID_ARG, "q8, k8 and v8 need scale arrays");
  if (q8->B != q->B || q8->H != q->H || q8->L != q->L || k8->B != k->B || k8->H != k->H || k8->L != k->L ||
      v8->B != v->B || v8->H != v->H || v8->L != v->L)
    return fail(FA_ERR_INVALID_ARG, "quantized outputs must have the shapes of their sources");
  if ((int64_t)q->B * q->H > 65535 || (int64_t)k->B * k->H > 65535 || q->B > 65535)
    return fail(FA_ERR_UNSUPPORTED, "B and H above the grid limits");
  // q_delta has one entry per query row: NULL is fine without rows.
  if (k_mean == nullptr ? q_delta != nullptr : (q_delta == nullptr && (int64_t)q->B * q->L > 0))
    return fail(FA_ERR_INVALID_ARG, "K centering needs both k_mean and q_delta (or neither)");
  if (q->H % k->H != 0) return fail(FA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", q->H, k->H);
  if (k_mean && (q->B != k->B)) return fail(FA_ERR_INVALID_ARG, "batch sizes differ");
  if ((reinterpret_cast<uintptr_t>(k_mean) & 3u) || (reinterpret_cast<uintptr_t>(q_delta) & 3u))
    return fail(FA_ERR_INVALID_ARG, "k_mean and q_delta must be 4-byte aligned");
  const int chunks = fa::quant_mean_chunks(k->L);
  if (k_mean) {
    const size_t need = flexattn_quantize_qkv_ex_workspace_bytes(k->B, k->H, k->L);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
      return fail(FA_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(FA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  fa::QuantArgs a{};
  a.qk_block = qk_block;
  a.k_mean = k_mean;
  a.q_delta = q_delta;
  a.mean_part = static_cast<double*>(workspace);
  a.mean_chunks = chunks;
  auto src = [](const fa_tensor* t) {
    return fa::QuantTensor{static_cast<const unsigned short*>(t->data), t->B, t->H, t->L, t->stride_b, t->stride_h, t->stride_l};
  };
  auto dst = [](fa_tensor* t, int nblocks) {
    return fa::QuantOut{static_cast<signed char*>(t->data), const_cast<float*>(t->scale), nblocks, t->stride_b,
                        t->stride_h, t->stride_l};
  };
  a.q = src(q);
  a.k = src(k);
  a.v = src(v);
  a.q8 = dst(q8, cdiv(q->L, qk_block));
  a.k8 = dst(k8, cdiv(k->L, qk_block));
  a.v8 = dst(v8, 128);
  if ((st = check_device()) != FA_OK) return st;
  hipError_t e = fa::launch_quantize(a, stream);
  if (e != hipSuccess) return fail(FA_ERR_DEVICE, "quantize launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status flexattn_quantize_qkv(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, fa_tensor* q8,
                                fa_tensor* k8, fa_tensor* v8, hipStream_t stream) {
  return quantize_impl(q, k, v, q8, k8, v8, 128, nullptr, nullptr, nullptr, 0, stream);
}

fa_status flexattn_quantize_qkv_ex(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, fa_tensor* q8,
                                   fa_tensor* k8, fa_tensor* v8, int qk_block, float* k_mean, float* q_delta,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return quantize_impl(q, k, v, q8, k8, v8, qk_block, k_mean, q_delta, workspace, workspace_bytes, stream);
}

static fa_status fwd_quantized(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_block_mask* bm,
                               int mask_kind, int score_kind, const fa_params* p, fa_tensor* out, float* lse,
                               int qk_block, const float* q_delta, hipStream_t stream) {
  fa_status st;
  if (qk_block != 128 && qk_block != 32) return fail(FA_ERR_UNSUPPORTED, "qk_block must be 128 or 32 (got %d)", qk_block);
  if (reinterpret_cast<uintptr_t>(q_delta) & 3u) return fail(FA_ERR_INVALID_ARG, "q_delta must be 4-byte aligned");
  if ((st = check_q_tensor(q, "q", FA_I8, 16)) != FA_OK) return st;
  if ((st = check_q_tensor(k, "k", FA_I8, 16)) != FA_OK) return st;
  if ((st = check_q_tensor(v, "v", FA_FP8_E4M3, 16)) != FA_OK) return st;
  if ((st = check_q_tensor(out, "out", FA_BF16, 8)) != FA_OK) return st;
  if (needs_scale(q, q->L) || needs_scale(k, k->L) || needs_scale(v, 1))
    return fail(FA_ERR_INVALID_ARG, "quantized q, k and v need scale arrays");
  if (out->scale) return fail(FA_ERR_INVALID_ARG, "out->scale must be NULL");
  if (mask_kind != FA_MASK_NONE || score_kind != FA_SCORE_NONE || bm != nullptr)
    return fail(FA_ERR_UNSUPPORTED, "the quantized form serves unmasked attention without score_mod (no BlockMask)");
  if (k->B != q->B || v->B != q->B || out->B != q->B) return fail(FA_ERR_INVALID_ARG, "batch sizes differ");
  if (k->H != v->H || k->L != v->L) return fail(FA_ERR_INVALID_ARG, "k and v shapes differ");
  if (q->H % k->H != 0) return fail(FA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", q->H, k->H);
  if (out->H != q->H || out->L != q->L) return fail(FA_ERR_INVALID_ARG, "out shape differs from q");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const int64_t total = (int64_t)q->B * q->H * cdiv(q->L, 128);
  if (total > 0x7fffffff) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  fa::QuantFwdArgs a{};
  a.q = static_cast<const signed char*>(q->data);
  a.k = static_cast<const signed char*>(k->data);
  a.v = static_cast<const unsigned char*>(v->data);
  a.o = static_cast<__bf16*>(out->data);
  a.lse = lse;
  a.q_sb = q->stride_b; a.q_sh = q->stride_h; a.q_sl = q->stride_l;
  a.k_sb = k->stride_b; a.k_sh = k->stride_h; a.k_sl = k->stride_l;
  a.v_sb = v->stride_b; a.v_sh = v->stride_h; a.v_sl = v->stride_l;
  a.o_sb = out->stride_b; a.o_sh = out->stride_h; a.o_sl = out->stride_l;
  a.q_scale = q->scale; a.k_scale = k->scale; a.v_scale = v->scale;
  a.B = q->B; a.Hq = q->H; a.Hkv = k->H; a.Lq = q->L; a.Lkv = k->L; a.group = q->H / k->H;
  a.nqb = cdiv(q->L, qk_block); a.nkb = cdiv(k->L, qk_block); a.nqw = cdiv(q->L, 128);
  a.qk_block = qk_block;
  a.q_delta = q_delta;
  const float sm = (p && p->sm_scale > 0.f) ? p->sm_scale : 1.0f / std::sqrt(128.0f);
  a.scale_log2 = sm * 1.4426950408889634f;
  a.sm_scale = sm;
  a.total_wg = (int)total;
  if ((st = check_device()) != FA_OK) return st;
  hipError_t e = fa::launch_fwd_quant(a, stream);
  if (e != hipSuccess) return fail(FA_ERR_DEVICE, "forward launch failed: %s", hipGetErrorString(e));
  return ok();
}



size_t flexattn_bwd_workspace_bytes(int B, int Hq, int Lq) {
  if (B < 0 || Hq < 0 || Lq < 0) return 0;
  const size_t rows = (size_t)B * Hq * Lq;
  const size_t rows4 = (rows + 3) / 4 * 4;  // keeps each part 16-byte aligned
  return (2 * rows4 + (size_t)B * Hq * cdiv(Lq, 128)) * sizeof(float);
}

fa_status flexattn_block_mask_transpose(const fa_block_mask* bm, fa_block_mask_transposed* out, hipStream_t stream) {
  if (bm == nullptr || out == nullptr) return fail(FA_ERR_INVALID_ARG, "bm and out must not be NULL");
  if (out->Bm != bm->Bm || out->Hm != bm->Hm || out->q_len != bm->q_len || out->kv_len != bm->kv_len ||
      out->q_block != bm->q_block || out->kv_block != bm->kv_block || out->n_qb != bm->n_qb || out->n_kvb != bm->n_kvb)
    return fail(FA_ERR_INVALID_ARG, "out's dimensions must equal the BlockMask's");
  if (bm->Bm <= 0 || bm->Hm <= 0 || bm->q_block <= 0 || bm->kv_block <= 0 || bm->q_len < 0 || bm->kv_len < 0 ||
      bm->n_qb != cdiv(bm->q_len, bm->q_block) || bm->n_kvb != cdiv(bm->kv_len, bm->kv_block))
    return fail(FA_ERR_INVALID_ARG, "BlockMask dimensions are inconsistent");
  if ((int64_t)bm->Bm * bm->Hm * bm->n_kvb > ((int64_t)1 << 31) - 4)
    return fail(FA_ERR_UNSUPPORTED, "too many BlockMask columns");
  if (bm->n_qb > 0 && bm->n_kvb > 0 &&
      (!bm->kv_num_blocks || !bm->full_kv_num_blocks || !bm->kv_indices || !bm->full_kv_indices))
    return fail(FA_ERR_INVALID_ARG, "BlockMask arrays are NULL");
  if (bm->n_kvb > 0 && (!out->q_num_blocks || !out->full_q_num_blocks || (bm->n_qb > 0 && (!out->q_indices || !out->full_q_indices))))
    return fail(FA_ERR_INVALID_ARG, "transposed BlockMask arrays are NULL");
  fa::TransposeArgs t{};
  t.Bm = bm->Bm;
  t.Hm = bm->Hm;
  t.nqb = bm->n_qb;
  t.nkvb = bm->n_kvb;
  t.kv_num = bm->kv_num_blocks;
  t.kv_idx = bm->kv_indices;
  t.full_num = bm->full_kv_num_blocks;
  t.full_idx = bm->full_kv_indices;
  t.q_num = out->q_num_blocks;
  t.q_idx = out->q_indices;
  t.fullq_num = out->full_q_num_blocks;
  t.fullq_idx = out->full_q_indices;
  if (reinterpret_cast<uintptr_t>(out->col_order) & 3u) return fail(FA_ERR_INVALID_ARG, "col_order must be 4-byte aligned");
  fa_status st = check_device();
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_block_mask_transpose(t, stream);
  if (e == hipSuccess && out->col_order && bm->n_kvb > 0) {
    fa::BlockMaskArgs o{};
    o.nqb = bm->n_kvb;  // the schedule kernel sorts rows of nqb entries: here columns
    o.full_num = out->full_q_num_blocks;
    o.kv_num = out->q_num_blocks;
    o.row_order = out->col_order;
    e = fa::launch_block_mask_order(o, bm->Bm * bm->Hm, stream);
  }
  if (e != hipSuccess) return fail(FA_ERR_DEVICE, "transpose launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status flexattn_bwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                       const fa_tensor* dout, const float* lse, const fa_block_mask* bm,
                       const fa_block_mask_transposed* bmt, int mask_kind, int score_kind, const fa_params* p,
                       fa_tensor* dq, fa_tensor* dk, fa_tensor* dv, float* dslopes, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !dout || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARG, "q, k, v, out, dout, dq, dk and dv must not be NULL");
  const fa_tensor* all[8] = {q, k, v, out, dout, dq, dk, dv};
  const char* names[8] = {"q", "k", "v", "out", "dout", "dq", "dk", "dv"};
  for (int i = 0; i < 8; ++i) {
    if (all[i]->dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "the backward serves bf16 tensors (%s)", names[i]);
    fa_status st = check_tensor(all[i], names[i], 8);
    if (st != FA_OK) return st;
    if (all[i]->D != 128) return fail(FA_ERR_UNSUPPORTED, "head dim must be 128 (%s has %d)", names[i], all[i]->D);
    if (all[i]->B != q->B) return fail(FA_ERR_INVALID_ARG, "batch sizes differ (%s)", names[i]);
  }
  if (k->H != v->H || k->L != v->L || dk->H != k->H || dk->L != k->L || dv->H != k->H || dv->L != k->L)
    return fail(FA_ERR_INVALID_ARG, "k, v, dk and dv must share one shape");
  if (out->H != q->H || out->L != q->L || dout->H != q->H || dout->L != q->L || dq->H != q->H || dq->L != q->L)
    return fail(FA_ERR_INVALID_ARG, "q, out, dout and dq must share one shape");
  if (q->H % k->H != 0) return fail(FA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", q->H, k->H);
  const int B = q->B, Hq = q->H, Lq = q->L, Lkv = k->L;
  if (lse == nullptr && (int64_t)B * Hq * Lq > 0) return fail(FA_ERR_INVALID_ARG, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  fa_status st;
  if ((st = check_mask(mask_kind, p, Lq, Lkv)) != FA_OK) return st;
  if (score_kind & ~kValidScore) return fail(FA_ERR_INVALID_ARG, "unknown score_kind bits 0x%x", score_kind);
  if (score_kind != FA_SCORE_NONE && p == nullptr) return fail(FA_ERR_INVALID_ARG, "params is NULL");
  if ((score_kind & FA_SCORE_ALIBI) && p->alibi_slopes == nullptr)
    return fail(FA_ERR_INVALID_ARG, "ALIBI needs alibi_slopes");
  if ((score_kind & FA_SCORE_SOFTCAP) && !(p->softcap > 0.f)) return fail(FA_ERR_INVALID_ARG, "SOFTCAP needs softcap > 0");
  if (dslopes != nullptr && !(score_kind & FA_SCORE_ALIBI))
    return fail(FA_ERR_INVALID_ARG, "dslopes is only written with ALIBI; pass NULL");
  if (reinterpret_cast<uintptr_t>(dslopes) & 3u) return fail(FA_ERR_INVALID_ARG, "dslopes must be 4-byte aligned");
  const int nqb = cdiv(Lq, 128), nkvb = cdiv(Lkv, 128);
  if ((int64_t)B * Hq * nqb > 0x7fffffff || (int64_t)B * k->H * nkvb > 0x7fffffff || Hq > 65535)
    return fail(FA_ERR_UNSUPPORTED, "grid too large");

  fa::BwdArgs a{};
  if (bm == nullptr || bmt == nullptr) {
    if (bm != nullptr || bmt != nullptr)
      return fail(FA_ERR_INVALID_ARG, "pass both the BlockMask and its transpose, or neither");
    if (mask_kind != FA_MASK_NONE) return fail(FA_ERR_INVALID_ARG, "a BlockMask is required unless mask_kind is NONE");
    a.all_full = 1;
    a.Bm = a.Hm = 1;
  } else {
    if (bm->q_len != Lq || bm->kv_len != Lkv)
      return fail(FA_ERR_INVALID_ARG, "BlockMask was built for lengths (%d, %d), not (%d, %d)", bm->q_len, bm->kv_len, Lq, Lkv);
    if (bm->q_block != 128 || bm->kv_block != 128)
      return fail(FA_ERR_UNSUPPORTED, "the backward needs 128 x 128 BlockMask tiles (got %d x %d)", bm->q_block, bm->kv_block);
    if (bm->n_qb != nqb || bm->n_kvb != nkvb)
      return fail(FA_ERR_INVALID_ARG, "BlockMask n_qb/n_kvb do not match its lengths and block sizes");
    if (bm->Bm != 1 && bm->Bm != B) return fail(FA_ERR_INVALID_ARG, "BlockMask Bm must be 1 or B");
    if (bm->Hm != 1) return fail(FA_ERR_UNSUPPORTED, "the backward needs a head-independent BlockMask (Hm = 1)");
    if (bmt->Bm != bm->Bm || bmt->Hm != bm->Hm || bmt->q_len != Lq || bmt->kv_len != Lkv || bmt->q_block != 128 ||
        bmt->kv_block != 128 || bmt->n_qb != nqb || bmt->n_kvb != nkvb)
      return fail(FA_ERR_INVALID_ARG, "the transposed BlockMask's dimensions differ from the BlockMask's");
    if (nqb > 0 && nkvb > 0 &&
        (!bm->kv_num_blocks || !bm->full_kv_num_blocks || !bm->kv_indices || !bm->full_kv_indices ||
         !bmt->q_num_blocks || !bmt->full_q_num_blocks || !bmt->q_indices || !bmt->full_q_indices))
      return fail(FA_ERR_INVALID_ARG, "BlockMask arrays are NULL");
    a.all_full = 0;
    a.Bm = bm->Bm;
    a.Hm = bm->Hm;
    a.row_order = bm->row_order;    // schedule of the dq pass
    a.col_order = bmt->col_order;   // schedule of the dk/dv pass
    a.kv_num = bm->kv_num_blocks;
    a.kv_idx = bm->kv_indices;
    a.full_num = bm->full_kv_num_blocks;
    a.full_idx = bm->full_kv_indices;
    a.q_num = bmt->q_num_blocks;
    a.q_idx = bmt->q_indices;
    a.fullq_num = bmt->full_q_num_blocks;
    a.fullq_idx = bmt->full_q_indices;
    if (verify_enabled()) {
      if ((st = verify_lists(bm->full_kv_num_blocks, bm->full_kv_indices, bm->kv_num_blocks, bm->kv_indices,
                             (int64_t)bm->Bm * bm->Hm * nqb, nkvb, "BlockMask", stream)) != FA_OK)
        return st;
      if ((st = verify_lists(bmt->full_q_num_blocks, bmt->full_q_indices, bmt->q_num_blocks, bmt->q_indices,
                             (int64_t)bmt->Bm * bmt->Hm * nkvb, nqb, "transposed BlockMask", stream)) != FA_OK)
        return st;
    }
  }
  const size_t need = flexattn_bwd_workspace_bytes(B, Hq, Lq);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(FA_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  a.q = q->data; a.k = k->data; a.v = v->data; a.o = out->data; a.dout = dout->data; a.lse = lse;
  a.dq = dq->data; a.dk = dk->data; a.dv = dv->data; a.dslopes = dslopes;
  a.q_sb = q->stride_b; a.q_sh = q->stride_h; a.q_sl = q->stride_l;
  a.k_sb = k->stride_b; a.k_sh = k->stride_h; a.k_sl = k->stride_l;
  a.v_sb = v->stride_b; a.v_sh = v->stride_h; a.v_sl = v->stride_l;
  a.o_sb = out->stride_b; a.o_sh = out->stride_h; a.o_sl = out->stride_l;
  a.do_sb = dout->stride_b; a.do_sh = dout->stride_h; a.do_sl = dout->stride_l;
  a.dq_sb = dq->stride_b; a.dq_sh = dq->stride_h; a.dq_sl = dq->stride_l;
  a.dk_sb = dk->stride_b; a.dk_sh = dk->stride_h; a.dk_sl = dk->stride_l;
  a.dv_sb = dv->stride_b; a.dv_sh = dv->stride_h; a.dv_sl = dv->stride_l;
  a.B = B; a.Hq = Hq; a.Hkv = k->H; a.Lq = Lq; a.Lkv = Lkv; a.group = Hq / k->H;
  a.nqb = nqb;
  a.nkvb = nkvb;
  a.flags = mask_kind;
  a.window = (mask_kind & FA_MASK_WINDOW) ? p->window : 0;
  a.prefix_len = (mask_kind & FA_MASK_PREFIX_LM) ? p->prefix_len : 0;
  a.q_doc = (mask_kind & FA_MASK_DOC) ? p->q_doc : nullptr;
  a.kv_doc = (mask_kind & FA_MASK_DOC) ? p->kv_doc : nullptr;
  a.sm_scale = (p && p->sm_scale > 0.f) ? p->sm_scale : 1.0f / std::sqrt((float)q->D);
  a.softcap = (score_kind & FA_SCORE_SOFTCAP) ? p->softcap : 0.f;
  a.inv_softcap = (score_kind & FA_SCORE_SOFTCAP) ? 1.0f / p->softcap : 0.f;
  a.slopes = (score_kind & FA_SCORE_ALIBI) ? p->alibi_slopes : nullptr;
  const size_t rows = (size_t)B * Hq * Lq, rows4 = (rows + 3) / 4 * 4;
  float* ws = static_cast<float*>(workspace);
  a.lse2 = ws;
  a.delta = ws ? ws + rows4 : nullptr;
  a.slope_part = (dslopes != nullptr && ws) ? ws + 2 * rows4 : nullptr;  // read only when rows > 0
  if ((st = check_device()) != FA_OK) return st;
  hipError_t e = fa::launch_bwd(a, score_kind, stream);
  if (e != hipSuccess) return fail(FA_ERR_DEVICE, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// BlockMask build for callers that cannot allocate (HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): flexattn_block_mask_build_noalloc is flexattn_block_mask_build
// with the builder's device scratch taken from a fixed static array instead of a caller
// workspace. It allocates nothing and runs the same kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "flexattn.h"

namespace {

// The builder's scratch: per-block document-id summaries, 16 bytes per query block and per kv
// block and batch (flexattn_block_mask_workspace_bytes). Each device holds its own copy of this
// array for the life of the process. On the host its name is only a stand-in for the symbol,
// never an address: the device address is read once per device with hipGetSymbolAddress, with
// that device current, kept in g_scratch_ptr, and only that pointer reaches the kernels. Every
// summary is written by the builder before it is read, so nothing needs clearing between calls.
// Calls that overlap on one device share the array and race.
constexpr size_t kScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[fa_api::kMaxDevices] = {};

// Device address of this device's scratch (resolved on the first call on the device).
fa_status scratch_ptr(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fa_api::fail(FA_ERR_DEVICE, "no current HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= fa_api::kMaxDevices)
    return fa_api::fail(FA_ERR_UNSUPPORTED, "device index %d above %d", dev, fa_api::kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fa_api::fail(FA_ERR_DEVICE, "cannot resolve the static scratch on device %d: %s", dev,
                          hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

size_t flexattn_block_mask_noalloc_max_bytes(void) { return kScratchBytes; }

fa_status flexattn_block_mask_build_noalloc(int mask_kind, const fa_params* p, int B, int q_len, int kv_len,
                                            fa_block_mask* out, hipStream_t stream) {
  fa_status st = fa_api::check_build(mask_kind, p, B, q_len, kv_len, out);
  if (st != FA_OK) return st;
  const size_t need = flexattn_block_mask_workspace_bytes(mask_kind, B, q_len, kv_len, out->q_block, out->kv_block);
  if (need > kScratchBytes)
    return fa_api::fail(FA_ERR_UNSUPPORTED,
                        "the builder's summaries need %zu bytes, above the %zu-byte static scratch of the "
                        "allocation-free entry point (use flexattn_block_mask_build with a workspace)",
                        need, kScratchBytes);
  if ((st = fa_api::check_device()) != FA_OK) return st;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_ptr(&ws)) != FA_OK) return st;
  return fa_api::launch_build(mask_kind, p, B, q_len, kv_len, out, ws, need, stream);
}

}  // extern "C"

// Helpers of the C-ABI layer (api.cpp) that other host sources of the library share: error
// reporting, the device-architecture check and the BlockMask builder's validation and launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "flexattn.h"

namespace fa_api {

constexpr int kMaxDevices = 64;  // device indices served (per-device caches)

// Record the reason of a non-OK status for flexattn_last_error() and return `st`.
fa_status fail(fa_status st, const char* fmt, ...);
fa_status ok();
// FA_ERR_UNSUPPORTED unless the current device is a gfx950 (see api.cpp).
fa_status check_device();
// Validation of a BlockMask build request (device and host builders).
fa_status check_build(int mask_kind, const fa_params* p, int B, int q_len, int kv_len, const fa_block_mask* out);
// Enqueue the device builder with `workspace` holding `need` bytes of per-block summaries.
fa_status launch_build(int mask_kind, const fa_params* p, int B, int q_len, int kv_len, fa_block_mask* out,
                       void* workspace, size_t need, hipStream_t stream);

}  // namespace fa_api

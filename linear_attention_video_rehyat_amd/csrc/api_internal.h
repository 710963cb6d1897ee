// api_internal.h -- entry points of api.cpp that other translation units of
// the library call (not part of the C ABI).
#pragma once

#include <stddef.h>

#include "../../include/rehyat.h"

namespace rehyat {

// rehyat_attn_fwd (bf16, recurrent partition) with its workspace in a fixed
// device buffer of `ws_bytes` bytes instead of the stream's arena: the same
// validation, kernels and results; REHYAT_ENOMEM if the call needs more.  Once
// the arguments are valid, get_ws supplies the buffer's device address for
// the current device (or an error status).
typedef rehyat_status (*fixed_workspace_fn)(char** ws);
rehyat_status fwd_fixed_workspace(const void* q, const void* k, const void* v, void* out, int B, int H,
                                  int frames, int tokens_per_frame, int head_dim, int chunk_frames,
                                  int overlap_frames, int feature_map, void* stream, fixed_workspace_fn get_ws,
                                  size_t ws_bytes);

// Records a HIP runtime failure (a hipError_t value) as the calling thread's
// last error and returns REHYAT_EHIP.
rehyat_status report_hip_error(int err, const char* what);

}  // namespace rehyat

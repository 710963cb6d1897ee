// noalloc.hip -- rehyat_attn_fwd_noalloc: the whole-clip forward with its
// workspace in a fixed, file-scope device array instead of an allocated
// arena, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives in every device's copy of this code object, at a different
// address on each device.  Its name is only a host-side stand-in: the device
// address comes from hipGetSymbolAddress, looked up once per device (with that
// device current) on the first call there and kept; kernels only ever receive
// that address.  Every call on a device shares the array, which keeps the last
// call's contents; the forward writes every workspace element it reads before
// reading it, so nothing needs clearing.  Calls that overlap on one device
// (concurrent streams, or threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "api_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<char*> g_scratch_ptr;  // per device: the array's device address (null: not looked up yet)

rehyat_status scratch_for_current_device(char** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return rehyat::report_hip_error(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return rehyat::report_hip_error(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = (char*)p;
    }
    *out = g_scratch_ptr[dev];
    return REHYAT_OK;
}

}  // namespace

extern "C" rehyat_status rehyat_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B,
                                                 int H, int frames, int tokens_per_frame, int head_dim,
                                                 int chunk_frames, int overlap_frames, int feature_map,
                                                 void* stream) {
    return rehyat::fwd_fixed_workspace(q, k, v, out, B, H, frames, tokens_per_frame, head_dim, chunk_frames,
                                       overlap_frames, feature_map, stream, scratch_for_current_device,
                                       kScratchBytes);
}

extern "C" size_t rehyat_noalloc_workspace_limit(void) { return kScratchBytes; }

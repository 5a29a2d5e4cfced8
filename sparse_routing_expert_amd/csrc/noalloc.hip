// moe_permute_noalloc: moe_permute without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The permute's scratch (per-tile expert counts and per-tile bases of the histogram/scan) lives
// in a fixed device array of this file instead of the caller's workspace. Each device holds its
// own copy of the array, at its own address, for the life of the process. The host-side name
// `scratch` is only a stand-in for that address: host code never passes it to a kernel or a copy,
// it passes the device address taken with hipGetSymbolAddress once per device (kept below).
//
// Every call on one device shares that device's array. Calls that overlap on one device (two
// streams, or two host threads) race on it; callers serialise them. Nothing in the array has to
// start at zero: each call writes every tile count before the scan or the scatter reads it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/moe.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, taken once per device.
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

inline bool ok_ptr(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int moe_permute_noalloc(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* offsets,
                                   int32_t* sorted_token, int32_t* inv_pos, void* x_perm, moe_stream_t stream) {
    // host checks first (shape, pointers, scratch size), so a rejected call makes no HIP call
    size_t need = 0;
    const int rc = moe_workspace_bytes(shape, MOE_STAGE_PERMUTE, &need);
    if (rc != MOE_OK) return rc;
    if (!(ok_ptr(topk_idx) && ok_ptr(x) && ok_ptr(offsets) && ok_ptr(sorted_token) && ok_ptr(inv_pos) &&
          (x_perm == nullptr || ok_ptr(x_perm))))
        return MOE_ERR_INVALID_ARG;
    if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
    if (shape->T == 0) return MOE_OK;
    void* ws = nullptr;
    const int rs = scratch_on_current_device(&ws);
    if (rs != MOE_OK) return rs;
    return moe_permute(shape, topk_idx, x, offsets, sorted_token, inv_pos, x_perm, ws, kScratchBytes, stream);
}

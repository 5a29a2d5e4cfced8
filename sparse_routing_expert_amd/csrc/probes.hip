// Measurement probes (include/moe_probe.h): what this card reaches on a plain streaming copy and on
// a loop of matrix instructions alone, run beside the layer so its fractions of the published peaks
// can be read against what is achievable on the same machine at the same moment. Not part of the
// layer.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/moe_probe.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// dst[i] = src[i] over n 16-byte vectors: each block copies 4096-vector chunks (64 KB), grid-stride
// over chunks; a thread issues its 16 loads of a chunk before its 16 stores, and each wave
// instruction moves 1 KB contiguous. Streaming (non-temporal) hints on both sides.
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                          int64_t n) {
    constexpr int U = 16, CH = 256 * U;
    for (int64_t c0 = (int64_t)blockIdx.x * CH; c0 < n; c0 += (int64_t)gridDim.x * CH) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = c0 + u * 256 + threadIdx.x;
            if (i < n) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = c0 + u * 256 + threadIdx.x;
            if (i < n) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

// iters x 8 independent v_mfma_f32_32x32x16_bf16 per wave on register operands; the accumulators
// are summed and written once per lane so the loop is not removed
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ out) {
    bf16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 7));
        b[i] = (__bf16)(0.002f * (float)((threadIdx.x + 3 * i) & 7));
    }
    floatx16_t acc[8];
    for (int j = 0; j < 8; ++j)
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
    for (int j = 0; j < 8; ++j)
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int moe_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
    if (src == nullptr || dst == nullptr || bytes <= 0 || (bytes & 15) || blocks <= 0) return -1;
    if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
    (void)hipGetLastError();
    probe_copy_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int moe_probe_mfma(int blocks, int iters, float* out, void* stream) {
    if (out == nullptr || blocks <= 0 || iters <= 0 || ((uintptr_t)out & 3)) return -1;
    (void)hipGetLastError();
    probe_mfma_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

double moe_probe_mfma_flops(int blocks, int iters) { return (double)blocks * 4.0 * iters * 8.0 * 32.0 * 32.0 * 16.0 * 2.0; }

}  // extern "C"

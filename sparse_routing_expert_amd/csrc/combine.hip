// moe_combine kernel: y[t] = sum_j g[t, j] * y_perm[inv_pos[t*k + j]] (+ y_shared[t])
// (Vector Institute post, Eq. (moe-output); "Router Optimization Techniques", MoE Layer Output;
// "Fine-tuning and serving MoE models", index_add of gate-scaled expert outputs).
//
// Token-major gather-reduce: one wave per token reads its k expert rows and the shared row with
// 128-bit loads (4 vectors per lane in flight, the next slot's rows loaded while the current one
// accumulates), accumulates in fp32 in slot order j = 0..k-1 (shared last) and rounds once. No
// atomics, so the result is deterministic.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe.h"

namespace moe {

template <bool BF16, int U>
__global__ __launch_bounds__(256) void combine_kernel(const uint8_t* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ topk_w,
                                                      const uint8_t* __restrict__ y_shared, uint8_t* __restrict__ y,
                                                      int64_t T, int d, int k) {
    constexpr int EB = BF16 ? 2 : 4;  // element bytes
    constexpr int EPV = 16 / EB;      // elements per 16-byte vector
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int mypos = lane < k ? inv_pos[t * k + lane] : 0;
    const float myg = lane < k ? topk_w[t * k + lane] : 0.f;
    const int64_t row_bytes = (int64_t)d * EB;
    const int nvec = d / EPV;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // U vectors per lane in flight; the rows of slot j + 1 are loaded while slot j accumulates
    for (int c0 = lane; c0 < nvec; c0 += 64 * U) {
        float acc[U][EPV];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < EPV; ++i) acc[u][i] = 0.f;
        u32x4 cur[U], nxt[U];
        {
            const int p = __builtin_amdgcn_readlane(mypos, 0);
            const uint8_t* row = y_perm + (int64_t)(p < 0 ? 0 : p) * row_bytes;
#pragma unroll
            for (int u = 0; u < U; ++u)
                cur[u] = p >= 0 && c0 + 64 * u < nvec ? ld16(row + (int64_t)(c0 + 64 * u) * 16) : zero;
        }
        for (int j = 0; j < k; ++j) {
            if (j + 1 < k) {
                const int p = __builtin_amdgcn_readlane(mypos, j + 1);
                const uint8_t* row = y_perm + (int64_t)(p < 0 ? 0 : p) * row_bytes;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    nxt[u] = p >= 0 && c0 + 64 * u < nvec ? ld16(row + (int64_t)(c0 + 64 * u) * 16) : zero;
            }
            // a slot dropped by expert capacity (row -1) adds nothing
            const bool kept = __builtin_amdgcn_readlane(mypos, j) >= 0;
            const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myg), j));
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[EPV];
                if (BF16) unpack8(cur[u], f);
                else
#pragma unroll
                    for (int i = 0; i < EPV; ++i) f[i] = __uint_as_float(cur[u][i]);
                if (kept)
#pragma unroll
                    for (int i = 0; i < EPV; ++i) acc[u][i] = fmaf(g, f[i], acc[u][i]);
                cur[u] = nxt[u];
            }
        }
        if (y_shared != nullptr) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                cur[u] = c0 + 64 * u < nvec ? ld16(y_shared + t * row_bytes + (int64_t)(c0 + 64 * u) * 16) : zero;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[EPV];
                if (BF16) unpack8(cur[u], f);
                else
#pragma unroll
                    for (int i = 0; i < EPV; ++i) f[i] = __uint_as_float(cur[u][i]);
#pragma unroll
                for (int i = 0; i < EPV; ++i) acc[u][i] += f[i];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + 64 * u >= nvec) break;
            u32x4 out;
            if (BF16) out = pack8(acc[u]);
            else
#pragma unroll
                for (int i = 0; i < EPV; ++i) out[i] = __float_as_uint(acc[u][i]);
            st16(y + t * row_bytes + (int64_t)(c0 + 64 * u) * 16, out);
        }
    }
}

void launch_combine(int dtype, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                    const void* y_shared, void* y, int64_t T, int d, int k, hipStream_t s) {
    const unsigned nblk = (unsigned)((T + 3) / 4);
    const auto yp = static_cast<const uint8_t*>(y_perm);
    const auto ys = static_cast<const uint8_t*>(y_shared);
    auto out = static_cast<uint8_t*>(y);
    if (dtype == MOE_BF16)
        combine_kernel<true, 4><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
    else
        combine_kernel<false, 4><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
}

}  // namespace moe

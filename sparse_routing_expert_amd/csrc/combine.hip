// moe_combine kernel: y[t] = sum_j g[t, j] * y_perm[inv_pos[t*k + j]] (+ y_shared[t])
// (Vector Institute post, Eq. (moe-output); "Router Optimization Techniques", MoE Layer Output;
// "Fine-tuning and serving MoE models", index_add of gate-scaled expert outputs).
//
// Token-major gather-reduce: one wave per token loads all k expert rows of its current column block
// (and the shared row) with 128-bit non-temporal loads before accumulating, so 16 to 32 vectors per
// lane are in flight; it accumulates in fp32 in slot order j = 0..k-1 (shared last), rounds once and
// writes with non-temporal stores. Every byte is touched once, so the non-temporal hint keeps the
// rows from displacing cached data (and the caches from writing back on their account). No atomics:
// the result is deterministic.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe.h"

namespace moe {

__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// KMAX >= k slots, W vectors per lane per slot and column block
template <bool BF16, int KMAX, int W>
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
    const int mypos = lane < k ? inv_pos[t * k + lane] : -1;
    const float myg = lane < k ? topk_w[t * k + lane] : 0.f;
    const int64_t row_bytes = (int64_t)d * EB;
    const int nvec = d / EPV;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int c0 = lane; c0 < nvec; c0 += 64 * W) {
        u32x4 v[KMAX][W], vs[W];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < k) {
                // a slot dropped by expert capacity (row -1) loads nothing and adds nothing
                const int p = __builtin_amdgcn_readlane(mypos, j);
                const uint8_t* row = y_perm + (int64_t)(p < 0 ? 0 : p) * row_bytes;
#pragma unroll
                for (int u = 0; u < W; ++u)
                    v[j][u] = p >= 0 && c0 + 64 * u < nvec ? ld16_nt(row + (int64_t)(c0 + 64 * u) * 16) : zero;
            }
        }
        if (y_shared != nullptr) {
#pragma unroll
            for (int u = 0; u < W; ++u)
                vs[u] = c0 + 64 * u < nvec ? ld16_nt(y_shared + t * row_bytes + (int64_t)(c0 + 64 * u) * 16) : zero;
        }
        float acc[W][EPV];
#pragma unroll
        for (int u = 0; u < W; ++u)
#pragma unroll
            for (int i = 0; i < EPV; ++i) acc[u][i] = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < k && __builtin_amdgcn_readlane(mypos, j) >= 0) {
                const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myg), j));
#pragma unroll
                for (int u = 0; u < W; ++u) {
                    float f[EPV];
                    if (BF16) unpack8(v[j][u], f);
                    else
#pragma unroll
                        for (int i = 0; i < EPV; ++i) f[i] = __uint_as_float(v[j][u][i]);
#pragma unroll
                    for (int i = 0; i < EPV; ++i) acc[u][i] = fmaf(g, f[i], acc[u][i]);
                }
            }
        }
        if (y_shared != nullptr) {
#pragma unroll
            for (int u = 0; u < W; ++u) {
                float f[EPV];
                if (BF16) unpack8(vs[u], f);
                else
#pragma unroll
                    for (int i = 0; i < EPV; ++i) f[i] = __uint_as_float(vs[u][i]);
#pragma unroll
                for (int i = 0; i < EPV; ++i) acc[u][i] += f[i];
            }
        }
#pragma unroll
        for (int u = 0; u < W; ++u) {
            if (c0 + 64 * u >= nvec) break;
            u32x4 out;
            if (BF16) out = pack8(acc[u]);
            else
#pragma unroll
                for (int i = 0; i < EPV; ++i) out[i] = __float_as_uint(acc[u][i]);
            st16_nt(y + t * row_bytes + (int64_t)(c0 + 64 * u) * 16, out);
        }
    }
}

// W: 16-byte vectors per lane per slot row and column block. Up to 8 slots take 4, so a 4 KB row
// (d = 2048) is one pass with 32 vectors per lane in flight: the Qwen3-shaped combine (k = 8) went
// from 134 to 108 us with 4 instead of 2, outputs bit-identical (the same products in the same order).
template <bool BF16>
void launch_combine_t(const uint8_t* yp, const int32_t* inv_pos, const float* topk_w, const uint8_t* ys, uint8_t* out,
                      int64_t T, int d, int k, hipStream_t s) {
    const unsigned nblk = (unsigned)((T + 3) / 4);
    if (k <= 2) combine_kernel<BF16, 2, 8><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
    else if (k <= 4) combine_kernel<BF16, 4, 4><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
    else if (k <= 8) combine_kernel<BF16, 8, 4><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
    else if (k <= 16) combine_kernel<BF16, 16, 1><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
    else combine_kernel<BF16, 32, 1><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
}

void launch_combine(int dtype, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                    const void* y_shared, void* y, int64_t T, int d, int k, hipStream_t s) {
    const auto yp = static_cast<const uint8_t*>(y_perm);
    const auto ys = static_cast<const uint8_t*>(y_shared);
    auto out = static_cast<uint8_t*>(y);
    if (dtype == MOE_BF16) launch_combine_t<true>(yp, inv_pos, topk_w, ys, out, T, d, k, s);
    else launch_combine_t<false>(yp, inv_pos, topk_w, ys, out, T, d, k, s);
}

}  // namespace moe

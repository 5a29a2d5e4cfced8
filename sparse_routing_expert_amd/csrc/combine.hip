// moe_combine kernel: y[t] = sum_j g[t, j] * y_perm[inv_pos[t*k + j]] (+ y_shared[t])
// (Vector Institute post, Eq. (moe-output); "Router Optimization Techniques", MoE Layer Output;
// "Fine-tuning and serving MoE models", index_add of gate-scaled expert outputs).
//
// Token-major gather-reduce: one wave per token reads its k expert rows and the shared row with
// 128-bit loads, accumulates in fp32 in slot order j = 0..k-1 (shared last) and rounds once. No
// atomics, so the result is deterministic.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint8_t* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ topk_w,
                                                      const uint8_t* __restrict__ y_shared, uint8_t* __restrict__ y,
                                                      int64_t T, int d, int k) {
    constexpr int EB = BF16 ? 2 : 4;       // element bytes
    constexpr int EPV = 16 / EB;           // elements per 16-byte vector
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int mypos = lane < k ? inv_pos[t * k + lane] : 0;
    const float myg = lane < k ? topk_w[t * k + lane] : 0.f;
    const int64_t row_bytes = (int64_t)d * EB;
    const int nvec = d / EPV;
    for (int c = lane; c < nvec; c += 64) {
        float acc[EPV];
#pragma unroll
        for (int i = 0; i < EPV; ++i) acc[i] = 0.f;
        for (int j = 0; j < k; ++j) {
            const int p = __builtin_amdgcn_readlane(mypos, j);
            const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myg), j));
            const u32x4 v = ld16(y_perm + (int64_t)p * row_bytes + (int64_t)c * 16);
            float f[EPV];
            if (BF16) unpack8(v, f);
            else
#pragma unroll
                for (int i = 0; i < EPV; ++i) f[i] = __uint_as_float(v[i]);
#pragma unroll
            for (int i = 0; i < EPV; ++i) acc[i] = fmaf(g, f[i], acc[i]);
        }
        if (y_shared != nullptr) {
            const u32x4 v = ld16(y_shared + t * row_bytes + (int64_t)c * 16);
            float f[EPV];
            if (BF16) unpack8(v, f);
            else
#pragma unroll
                for (int i = 0; i < EPV; ++i) f[i] = __uint_as_float(v[i]);
#pragma unroll
            for (int i = 0; i < EPV; ++i) acc[i] += f[i];
        }
        u32x4 out;
        if (BF16) out = pack8(acc);
        else
#pragma unroll
            for (int i = 0; i < EPV; ++i) out[i] = __float_as_uint(acc[i]);
        st16(y + t * row_bytes + (int64_t)c * 16, out);
    }
}

void launch_combine(int dtype, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                    const void* y_shared, void* y, int64_t T, int d, int k, hipStream_t s) {
    const unsigned nblk = (unsigned)((T + 3) / 4);
    const auto yp = static_cast<const uint8_t*>(y_perm);
    const auto ys = static_cast<const uint8_t*>(y_shared);
    auto out = static_cast<uint8_t*>(y);
    if (dtype == MOE_BF16)
        combine_kernel<true><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
    else
        combine_kernel<false><<<nblk, 256, 0, s>>>(yp, inv_pos, topk_w, ys, out, T, d, k);
}

}  // namespace moe

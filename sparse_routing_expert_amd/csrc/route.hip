// moe_route kernels: router logits, scores, per-token top-k, gates, counts and balance statistics.
//
// Router (Vector Institute post, router score and softmax; "Router Optimization Techniques",
// What Is It?: h(x) = x W_g, TopK, Softmax(TopK(h)); How It Works 2: the bias only enters the
// top-k key). The router stays in fp32 ("Mixture of Experts" tutorial, Selective precision):
// bf16 activations are exact in fp32, and the fp32 router weights are split into three bf16
// terms (hi + mid + lo covers the 24-bit significand) so the logits run on the bf16 matrix cores
// with fp32 accumulation at fp32 accuracy.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe.h"

namespace moe {

namespace {

__device__ __forceinline__ void split3(const float* w, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        __bf16 h = (__bf16)w[j];
        float r1 = w[j] - (float)h;
        __bf16 m = (__bf16)r1;
        float r2 = r1 - (float)m;
        hi[j] = h;
        mid[j] = m;
        lo[j] = (__bf16)r2;
    }
}

// Order-preserving 64-bit key: larger float first, then the LOWER expert index (its complement
// sits in the low word), so one unsigned max gives the (key desc, index asc) total order.
__device__ __forceinline__ uint64_t pack_key(float v, int e) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

__device__ __forceinline__ float sigmoidf_(float l) { return 1.0f / (1.0f + expf(-l)); }

}  // namespace

// logits[T, E] = x[T, d] (bf16) . w[E, d]^T (fp32), one wave per 16 tokens x 16 experts
// (v_mfma_f32_16x16x32_bf16). Any assignment of the reduced index k to lanes is valid as long
// as both operands use the same one, so each lane reads 32 contiguous bf16 of its token row and
// the matching 32 fp32 of its expert row per 128-wide step: 64-byte contiguous loads.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void route_logits_bf16_kernel(const uint16_t* __restrict__ x,
                                                                       const float* __restrict__ w,
                                                                       float* __restrict__ logits, int64_t T,
                                                                       int d, int E) {
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int64_t t0 = ((int64_t)blockIdx.x * WAVES + wave) * 16;
    if (t0 >= T) return;  // no barriers in this kernel
    const int e0 = blockIdx.y * 16;
    const int r = lane & 15, g = lane >> 4;
    const int64_t t = t0 + r < T ? t0 + r : T - 1;
    const int e = e0 + r;
    const bool e_ok = e < E;
    const uint16_t* xr = x + t * d;
    const float* wr = w + (int64_t)(e_ok ? e : E - 1) * d;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int kb = 0;
    for (; kb + 128 <= d; kb += 128) {
        const int base = kb + g * 32;
        u32x4 xv[4];
        floatx4 wv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = ld16(xr + base + i * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[i] = *reinterpret_cast<const floatx4*>(wr + base + i * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float wf[8] = {wv[2 * i][0], wv[2 * i][1], wv[2 * i][2], wv[2 * i][3],
                           wv[2 * i + 1][0], wv[2 * i + 1][1], wv[2 * i + 1][2], wv[2 * i + 1][3]};
            if (!e_ok) {
#pragma unroll
                for (int j = 0; j < 8; ++j) wf[j] = 0.f;
            }
            bf16x8 hi, mid, lo;
            split3(wf, hi, mid, lo);
            const bf16x8 a = __builtin_bit_cast(bf16x8, xv[i]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, mid, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, acc, 0, 0, 0);
        }
    }
    for (; kb < d; kb += 32) {  // d is a multiple of 64: at most one 64-wide tail (two steps)
        const int base = kb + g * 8;
        const u32x4 xv = ld16(xr + base);
        const floatx4 w0 = *reinterpret_cast<const floatx4*>(wr + base);
        const floatx4 w1 = *reinterpret_cast<const floatx4*>(wr + base + 4);
        float wf[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
        if (!e_ok) {
#pragma unroll
            for (int j = 0; j < 8; ++j) wf[j] = 0.f;
        }
        bf16x8 hi, mid, lo;
        split3(wf, hi, mid, lo);
        const bf16x8 a = __builtin_bit_cast(bf16x8, xv);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, mid, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, acc, 0, 0, 0);
    }
    // 16x16 accumulator: lane holds column (expert) lane%16, rows (tokens) 4*(lane/16) + v.
    if (e_ok) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t tt = t0 + 4 * g + v;
            if (tt < T) logits[tt * E + e] = acc[v];
        }
    }
}

// fp32 activations: one thread per logit, sequential fp32 fused multiply-adds over d.
__global__ __launch_bounds__(256) void route_logits_f32_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               float* __restrict__ logits, int64_t T, int d,
                                                               int E) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T * E) return;
    const int64_t t = i / E;
    const int e = (int)(i - t * E);
    const floatx4* xr = reinterpret_cast<const floatx4*>(x + t * d);
    const floatx4* wr = reinterpret_cast<const floatx4*>(w + (int64_t)e * d);
    float acc = 0.f;
    for (int q = 0; q < d / 4; ++q) {
        const floatx4 a = xr[q], b = wr[q];
        acc = fmaf(a[0], b[0], acc);
        acc = fmaf(a[1], b[1], acc);
        acc = fmaf(a[2], b[2], acc);
        acc = fmaf(a[3], b[3], acc);
    }
    logits[i] = acc;
}

// Per token (one wave): scores, balance-statistic partials, top-k by k rounds of a wave-wide
// max over packed keys, gates. Each block (4 waves x 16 tokens) writes its expert histogram, its
// per-expert probability sums and its entropy sum; route_finalize reduces them in a fixed order.
template <int EPL>
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ logits,
                                                           const float* __restrict__ sel_bias, int64_t T,
                                                           int E, int k, int score, int renorm,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w,
                                                           int32_t* __restrict__ blk_counts,
                                                           float* __restrict__ blk_P, float* __restrict__ blk_H) {
    __shared__ int s_cnt[1024];
    __shared__ float s_P[4][1024];
    __shared__ float s_H[4];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = 0;
    __syncthreads();

    const bool softmax = score == MOE_SOFTMAX;
    float pacc[EPL], bias[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        pacc[i] = 0.f;
        bias[i] = (sel_bias != nullptr && e < E) ? sel_bias[e] : 0.f;
    }
    float hacc = 0.f;

    const int64_t tb = (int64_t)blockIdx.x * kRouteTokensPerBlock + wave * 16;
    for (int q = 0; q < 16; ++q) {
        const int64_t t = tb + q;
        if (t >= T) break;
        const float* lt = logits + t * E;
        float l[EPL];
        float lmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            l[i] = e < E ? lt[e] : -INFINITY;
            lmax = fmaxf(lmax, l[i]);
        }
        const float m = wave_max(lmax);
        // distribution whose mean is P_e and whose entropy is reported
        float p[EPL];
        float zpart = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            p[i] = e < E ? (softmax ? expf(l[i] - m) : sigmoidf_(l[i])) : 0.f;
            zpart += p[i];
        }
        const float Z = wave_sum(zpart);
        const float invZ = 1.0f / Z, lnZ = logf(Z);
        uint64_t key[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            const float pi = p[i] * invZ;
            pacc[i] += pi;
            if (pi > 0.f) hacc -= pi * (softmax ? (l[i] - m) - lnZ : logf(pi));
            float kv = softmax ? l[i] : p[i];  // p[i] holds the raw sigmoid score here
            kv = kv + bias[i];
            kv = kv + 0.0f;  // -0 -> +0: equal keys compare equal
            key[i] = e < E ? pack_key(kv, e) : 0ull;
        }
        int sel_e = 0;
        for (int j = 0; j < k; ++j) {
            uint64_t best = 0ull;
#pragma unroll
            for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
            best = wave_max_u64(best);
            const int e = key_index(best);
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (e == lane + 64 * i) key[i] = 0ull;
            if (lane == j) sel_e = e;
        }
        // gates from the unbiased logits of the selection (lane j holds slot j)
        const float lv = lane < k ? lt[sel_e] : -INFINITY;
        float gate;
        if (softmax) {
            if (renorm) {
                const float ms = wave_max(lv);
                const float ex = lane < k ? expf(lv - ms) : 0.f;
                gate = ex / wave_sum(ex);
            } else {
                gate = expf(lv - m) * invZ;
            }
        } else {
            const float s = lane < k ? sigmoidf_(lv) : 0.f;
            gate = s / wave_sum(s);
        }
        if (lane < k) {
            topk_idx[t * k + lane] = sel_e;
            topk_w[t * k + lane] = gate;
            atomicAdd(&s_cnt[sel_e], 1);
        }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) s_P[wave][e] = pacc[i];
    }
    const float hw = wave_sum(hacc);
    if (lane == 0) s_H[wave] = hw;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        blk_counts[(int64_t)blockIdx.x * E + e] = s_cnt[e];
        blk_P[(int64_t)blockIdx.x * E + e] = ((s_P[0][e] + s_P[1][e]) + s_P[2][e]) + s_P[3][e];
    }
    if (threadIdx.x == 0) blk_H[blockIdx.x] = ((s_H[0] + s_H[1]) + s_H[2]) + s_H[3];
}

// Fixed-order reduction of the per-block partials: counts, f = counts/T, P = mean p,
// aux = E * sum f P, mean entropy.
__global__ __launch_bounds__(256) void route_finalize_kernel(const int32_t* __restrict__ blk_counts,
                                                             const float* __restrict__ blk_P,
                                                             const float* __restrict__ blk_H, int nblk,
                                                             int64_t T, int E, int32_t* __restrict__ counts,
                                                             float* __restrict__ stats) {
    __shared__ double s_fp[1024];
    const double invT = 1.0 / (double)T;
    for (int e = threadIdx.x; e < E; e += 256) {
        int64_t c = 0;
        double P = 0.0;
        for (int b = 0; b < nblk; ++b) {
            c += blk_counts[(int64_t)b * E + e];
            P += (double)blk_P[(int64_t)b * E + e];
        }
        counts[e] = (int32_t)c;
        const double f = (double)c * invT, Pm = P * invT;
        s_fp[e] = f * Pm;
        if (stats) {
            stats[e] = (float)f;
            stats[E + e] = (float)Pm;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0 && stats) {
        double aux = 0.0, H = 0.0;
        for (int e = 0; e < E; ++e) aux += s_fp[e];
        for (int b = 0; b < nblk; ++b) H += (double)blk_H[b];
        stats[2 * E] = (float)(E * aux);
        stats[2 * E + 1] = (float)(H * invT);
    }
}

void launch_route_logits(int dtype, const void* x, const float* w_router, float* logits, int64_t T, int d,
                         int E, hipStream_t s) {
    if (dtype == MOE_BF16) {
        constexpr int W = 4;
        dim3 grid((unsigned)((T + 16 * W - 1) / (16 * W)), (unsigned)((E + 15) / 16));
        route_logits_bf16_kernel<W><<<grid, 64 * W, 0, s>>>(static_cast<const uint16_t*>(x), w_router, logits,
                                                            T, d, E);
    } else {
        const int64_t n = T * E;
        route_logits_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<const float*>(x),
                                                                           w_router, logits, T, d, E);
    }
}

void launch_route_select(const float* logits, const float* sel_bias, int64_t T, int E, int k, int score,
                         int renorm, int32_t* topk_idx, float* topk_w, int32_t* blk_counts, float* blk_P,
                         float* blk_H, hipStream_t s) {
    const unsigned nblk = (unsigned)((T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock);
#define MOE_SELECT(EPL)                                                                                  \
    route_select_kernel<EPL><<<nblk, 256, 0, s>>>(logits, sel_bias, T, E, k, score, renorm, topk_idx, topk_w, \
                                                 blk_counts, blk_P, blk_H)
    if (E <= 64) MOE_SELECT(1);
    else if (E <= 128) MOE_SELECT(2);
    else if (E <= 256) MOE_SELECT(4);
    else if (E <= 512) MOE_SELECT(8);
    else MOE_SELECT(16);
#undef MOE_SELECT
}

void launch_route_finalize(const int32_t* blk_counts, const float* blk_P, const float* blk_H, int nblk,
                           int64_t T, int E, int32_t* counts, float* stats, hipStream_t s) {
    route_finalize_kernel<<<1, 256, 0, s>>>(blk_counts, blk_P, blk_H, nblk, T, E, counts, stats);
}

}  // namespace moe

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

// Order-preserving 64-bit key: larger float first, then the LOWER expert index (its complement
// sits in the low word), so one unsigned max gives the (key desc, index asc) total order.
__device__ __forceinline__ uint64_t pack_key(float v, int e) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

__device__ __forceinline__ float sigmoidf_(float l) { return 1.0f / (1.0f + expf(-l)); }
__device__ __forceinline__ float softplusf_(float z) { return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))); }

}  // namespace

// Split of the fp32 router into three bf16 terms, once per call: w = hi + mid + lo with each term
// the bf16 rounding of what the previous ones leave, which carries the 24-bit significand. Rows
// E..Epad-1 are zero. The same launch zeroes the ticket route_finalize counts its blocks with.
__global__ __launch_bounds__(256) void route_prep_kernel(const float* __restrict__ w, int E, int Epad, int d,
                                                         uint16_t* __restrict__ wsplit, int32_t* __restrict__ ticket) {
    const int64_t n = (int64_t)Epad * d;
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (blockIdx.x == 0 && threadIdx.x == 0) *ticket = 0;
    if (wsplit == nullptr || i4 >= n) return;
    const int64_t row = i4 / d;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < E) v = *reinterpret_cast<const floatx4*>(w + i4);
    uint16_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const __bf16 h = (__bf16)v[j];
        const float r1 = v[j] - (float)h;
        const __bf16 m = (__bf16)r1;
        const float r2 = r1 - (float)m;
        const __bf16 l = (__bf16)r2;
        hi[j] = __builtin_bit_cast(uint16_t, h);
        mid[j] = __builtin_bit_cast(uint16_t, m);
        lo[j] = __builtin_bit_cast(uint16_t, l);
    }
    uint2 ph, pm, pl;
    ph.x = hi[0] | ((uint32_t)hi[1] << 16);
    ph.y = hi[2] | ((uint32_t)hi[3] << 16);
    pm.x = mid[0] | ((uint32_t)mid[1] << 16);
    pm.y = mid[2] | ((uint32_t)mid[3] << 16);
    pl.x = lo[0] | ((uint32_t)lo[1] << 16);
    pl.y = lo[2] | ((uint32_t)lo[3] << 16);
    *reinterpret_cast<uint2*>(wsplit + i4) = ph;
    *reinterpret_cast<uint2*>(wsplit + n + i4) = pm;
    *reinterpret_cast<uint2*>(wsplit + 2 * n + i4) = pl;
}

// logits[T, E] = x[T, d] (bf16) . w[E, d]^T with the split router (v_mfma_f32_16x16x32_bf16, three
// products per K step). A block owns 16*TT tokens x 16 experts; its NW waves take 1/NW of d each
// (TT token tiles per wave share each router load) and their partial tiles are summed in LDS in a
// fixed order. Each 32-wide K chunk of a 128-wide step is one load instruction per operand, in
// which the four lanes of a row read 64 contiguous bytes; the next step's loads are issued before
// the current products. NTX: x is read by one block only (E <= 16), so its loads are non-temporal.
template <int TT, bool NTX, int NW>
__global__ __launch_bounds__(NW * 64) void route_logits_bf16_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ wsplit, int Epad,
                                                                    float* __restrict__ logits, int64_t T, int d,
                                                                    int E) {
    __shared__ floatx4 s_part[NW][TT][64];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * 16 * TT;
    const int e0 = blockIdx.y * 16;
    const int r = lane & 15, g = lane >> 4;
    const uint16_t* xr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int64_t t = t0 + tt * 16 + r;
        xr[tt] = x + (t < T ? t : T - 1) * d;
    }
    const bool w_ok = e0 + r < E;  // rows E..Epad-1 are zero: not loaded
    const int64_t n = (int64_t)Epad * d;
    const uint16_t* wh = wsplit + (int64_t)(e0 + r) * d;
    const int nc = d / 32;  // 32-wide K chunks, split over the waves
    const int kb0 = (wave * nc / NW) * 32, kb1 = ((wave + 1) * nc / NW) * 32;
    floatx4 acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 xv[2][TT][4], wv[2][3][4];
#define RL_LOAD(b_, kb_)                                                                                  \
    {                                                                                                     \
        const int base = (kb_) + g * 8;                                                                   \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                   \
            _Pragma("unroll") for (int tt = 0; tt < TT; ++tt) xv[b_][tt][i] = NTX ?                       \
                __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr[tt] + base + i * 32)) :      \
                ld16(xr[tt] + base + i * 32);                                                             \
            _Pragma("unroll") for (int p = 0; p < 3; ++p) wv[b_][p][i] =                                   \
                w_ok ? ld16(wh + p * n + base + i * 32) : zero;                                           \
        }                                                                                                 \
    }
#define RL_MMA(b_)                                                                                        \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) _Pragma("unroll") for (int tt = 0; tt < TT; ++tt)      \
        _Pragma("unroll") for (int p = 0; p < 3; ++p) acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(   \
            __builtin_bit_cast(bf16x8, xv[b_][tt][i]), __builtin_bit_cast(bf16x8, wv[b_][p][i]), acc[tt], 0, 0, 0);
    int kb = kb0;
    const int nsteps = (kb1 - kb0) / 128;
    if (nsteps > 0) {
        RL_LOAD(0, kb)
        int st = 0;
        for (; st + 2 <= nsteps; st += 2) {
            if (st + 1 < nsteps) RL_LOAD(1, kb + 128)
            RL_MMA(0)
            if (st + 2 < nsteps) RL_LOAD(0, kb + 256)
            RL_MMA(1)
            kb += 256;
        }
        if (st < nsteps) {
            RL_MMA(0)
            kb += 128;
        }
    }
#undef RL_LOAD
#undef RL_MMA
    for (; kb < kb1; kb += 32) {  // 32-wide tail of the wave's range
        const int base = kb + g * 8;
        u32x4 w3[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) w3[p] = w_ok ? ld16(wh + p * n + base) : zero;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(xr[tt] + base));
#pragma unroll
            for (int p = 0; p < 3; ++p)
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, w3[p]), acc[tt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) s_part[wave][tt][lane] = acc[tt];
    __syncthreads();
    if (wave != 0) return;
    // 16x16 accumulator: lane holds column (expert) lane%16, rows (tokens) 4*(lane/16) + v.
    const int e = e0 + r;
    if (e < E) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            floatx4 sum = s_part[0][tt][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) sum += s_part[w][tt][lane];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t tk = t0 + tt * 16 + 4 * g + v;
                if (tk < T) logits[tk * E + e] = sum[v];
            }
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

// One token's selection, with its logits held as l[i] = logit of expert lane + 64 i (-inf past E):
// the scores' distribution (softmax or normalised sigmoid) is added to pacc and its entropy to
// hacc; the top-k by k rounds of a wave-wide max over packed (key, index) pairs, key = logit
// (softmax) or sigmoid score, plus the selection bias; the gates from the unbiased scores of the
// selection; slot j is written by lane j, which also counts its expert in s_cnt.
template <int EPL>
__device__ __forceinline__ void select_token(const float (&l)[EPL], const float (&bias)[EPL], int64_t t, int E,
                                             int k, bool softmax, int renorm, float (&pacc)[EPL], float& hacc,
                                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                             int* s_cnt) {
    const int lane = lane_id();
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) lmax = fmaxf(lmax, l[i]);
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
    float sel_l = -INFINITY;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = key_index(best);  // wave-uniform
        // unbiased logit of the winner, read from the lane that holds it
        float le = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if ((e >> 6) == i) le = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l[i]), e & 63));
            if (e == lane + 64 * i) key[i] = 0ull;
        }
        if (lane == j) {
            sel_e = e;
            sel_l = le;
        }
    }
    // gates from the unbiased logits of the selection (lane j holds slot j)
    const float lv = lane < k ? sel_l : -INFINITY;
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
        const float sg = lane < k ? sigmoidf_(lv) : 0.f;
        gate = sg / wave_sum(sg);
    }
    if (lane < k) {
        topk_idx[t * k + lane] = sel_e;
        topk_w[t * k + lane] = gate;
        atomicAdd(&s_cnt[sel_e], 1);
    }
}

// Per token (one wave per token, sixteen waves per block): scores, balance-statistic partials,
// top-k by k rounds of a wave-wide max over packed keys, gates. Each
// block writes its expert histogram, its per-expert probability sums and its entropy sum;
// route_finalize reduces them. Noisy top-k ("Mixture of Experts" tutorial, Noisy top-k gating):
// with s_logits (= x W_noise^T) and noise given, the logits become H = l + noise * softplus(s)
// before anything else, and H is written to h_out when that is given.
constexpr int kSelTokensPerWave = 1;
constexpr int kSelWaves = kRouteTokensPerBlock / kSelTokensPerWave;
template <int EPL>
__global__ __launch_bounds__(kSelWaves * 64) void route_select_kernel(const float* __restrict__ logits, int lg_ld,
                                                           int lg_split, float* __restrict__ logits_out,
                                                           const float* __restrict__ sel_bias, int64_t T,
                                                           int E, int k, int score, int renorm,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w,
                                                           int32_t* __restrict__ blk_counts,
                                                           float* __restrict__ blk_P, float* __restrict__ blk_H,
                                                           const float* __restrict__ s_logits,
                                                           const float* __restrict__ noise,
                                                           float* __restrict__ h_out) {
    __shared__ int s_cnt[64 * EPL];
    __shared__ float s_P[kSelWaves][64 * EPL];
    __shared__ float s_H[kSelWaves];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < E; e += kSelWaves * 64) s_cnt[e] = 0;
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

    const int64_t tb = (int64_t)blockIdx.x * kRouteTokensPerBlock + wave * kSelTokensPerWave;
    // logits of token t, expert e: lg[t * lg_ld + e], or with lg_split > 0 the sum of the three
    // split-router products (hi, mid, lo) at columns e, lg_split + e and 2 * lg_split + e
    auto logit_at = [&](const float* lg, int64_t t, int e) {
        const float* r = lg + t * lg_ld + e;
        return lg_split > 0 ? (r[0] + r[lg_split]) + r[2 * lg_split] : r[0];
    };
    float lall[kSelTokensPerWave][EPL];
#pragma unroll
    for (int q = 0; q < kSelTokensPerWave; ++q)
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            lall[q][i] = (tb + q < T && e < E) ? logit_at(logits, tb + q, e) : -INFINITY;
        }
    if (s_logits != nullptr) {
#pragma unroll
        for (int q = 0; q < kSelTokensPerWave; ++q)
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + 64 * i;
                if (tb + q < T && e < E) {
                    const int64_t o = (tb + q) * E + e;
                    lall[q][i] = lall[q][i] + noise[o] * softplusf_(logit_at(s_logits, tb + q, e));
                    if (h_out != nullptr) h_out[o] = lall[q][i];
                }
            }
    } else if (logits_out != nullptr) {
#pragma unroll
        for (int q = 0; q < kSelTokensPerWave; ++q)
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + 64 * i;
                if (tb + q < T && e < E) logits_out[(tb + q) * E + e] = lall[q][i];
            }
    }
#pragma unroll
    for (int q = 0; q < kSelTokensPerWave; ++q) {
        const int64_t t = tb + q;
        if (t >= T) break;
        select_token<EPL>(lall[q], bias, t, E, k, softmax, renorm, pacc, hacc, topk_idx, topk_w, s_cnt);
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) s_P[wave][e] = pacc[i];
    }
    const float hw = wave_sum(hacc);
    if (lane == 0) s_H[wave] = hw;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kSelWaves * 64) {
        blk_counts[(int64_t)blockIdx.x * E + e] = s_cnt[e];
        if (blk_P != nullptr) {
            float sp = s_P[0][e];
#pragma unroll
            for (int w = 1; w < kSelWaves; ++w) sp += s_P[w][e];
            blk_P[(int64_t)blockIdx.x * E + e] = sp;
        }
    }
    if (threadIdx.x == 0 && blk_H != nullptr) {
        float sh = s_H[0];
#pragma unroll
        for (int w = 1; w < kSelWaves; ++w) sh += s_H[w];
        blk_H[blockIdx.x] = sh;
    }
}

// Single-block form for routers of at most kFinalizeSmallExperts experts: item i <= E (expert i, or
// the entropy for i = E) goes to wave i % NWV; lane j of that wave sums blocks j, j + 64, ... in
// order and the wave adds its lanes in a fixed tree (float64 for the statistics). Thread 0 then forms
// aux = E * sum_e f_e P_e in expert order. One launch and no cross-block ticket.
constexpr int kFinalizeSmallExperts = 16;
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int lo = __shfl_xor(__double2loint(v), o), hi = __shfl_xor(__double2hiint(v), o);
        const double u = __hiloint2double(hi, lo);
        // the lane with the lower index keeps its own value on the left, so both lanes of a pair
        // form the same sum
        v = (lane_id() & o) ? u + v : v + u;
    }
    return v;
}
template <int NWV>
__device__ __forceinline__ void finalize_small_block(const int32_t* __restrict__ blk_counts,
                                                     const float* __restrict__ blk_P, const float* __restrict__ blk_H,
                                                     int nblk, int64_t T, int E, int32_t* __restrict__ counts,
                                                     float* __restrict__ stats, double* s_fp) {
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const double invT = 1.0 / (double)T;
    for (int it = wave; it <= E; it += NWV) {
        if (it < E) {
            int cnt = 0;
            double acc = 0.0;
            for (int b = lane; b < nblk; b += 64) {
                cnt += blk_counts[(int64_t)b * E + it];
                if (stats) acc += (double)blk_P[(int64_t)b * E + it];
            }
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o);
            if (stats) acc = wave_sum_f64(acc);
            if (lane == 0) {
                counts[it] = cnt;
                if (stats) {
                    const double f = (double)cnt * invT, Pm = acc * invT;
                    stats[it] = (float)f;
                    stats[E + it] = (float)Pm;
                    s_fp[it] = f * Pm;
                }
            }
        } else if (stats) {
            double acc = 0.0;
            for (int b = lane; b < nblk; b += 64) acc += (double)blk_H[b];
            acc = wave_sum_f64(acc);
            if (lane == 0) stats[2 * E + 1] = (float)(acc * invT);
        }
    }
    if (stats == nullptr) return;
    __syncthreads();
    if (threadIdx.x == 0) {
        double a = 0.0;
        for (int e = 0; e < E; ++e) a += s_fp[e];
        stats[2 * E] = (float)((double)E * a);
    }
}
__global__ __launch_bounds__(1024) void route_finalize_small_kernel(const int32_t* __restrict__ blk_counts,
                                                                    const float* __restrict__ blk_P,
                                                                    const float* __restrict__ blk_H, int nblk,
                                                                    int64_t T, int E, int32_t* __restrict__ counts,
                                                                    float* __restrict__ stats) {
    __shared__ double s_fp[kFinalizeSmallExperts];
    finalize_small_block<16>(blk_counts, blk_P, blk_H, nblk, T, E, counts, stats, s_fp);
}

// Small routers (E <= 16), bf16 activations: logits and selection in one launch. A block owns
// 16 * TT tokens and the 16 (padded) experts; its waves split d as in route_logits_bf16_kernel,
// but form the hi + mid + lo bf16 terms of the fp32 router in registers from fp32 loads (the same
// roundings as route_prep_kernel, so the products and their order are the same). The wave partials
// are summed in LDS in wave order, then each wave selects for its share of the block's tokens
// (select_token, lane e holding expert e) and the block writes its partials for route_finalize.
// NOISY (noisy top-k gating, "Mixture of Experts" tutorial, Noisy top-k gating): the K loop runs a
// second time with the noise-scale projection w_noise, and the selection uses
// H = l + noise * softplus(x w_noise^T) in place of l (H is what logits_out receives).
constexpr int kFusedRouteWaves = 8;
template <int TT, bool NOISY>
__global__ __launch_bounds__(kFusedRouteWaves * 64) void route_fused_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w, const float* __restrict__ w_noise,
    const float* __restrict__ noise, const float* __restrict__ sel_bias, int64_t T, int d, int E, int k, int score,
    int renorm, float* __restrict__ logits_out, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ blk_counts, float* __restrict__ blk_P, float* __restrict__ blk_H,
    int32_t* __restrict__ ticket) {
    constexpr int NW = kFusedRouteWaves, TPB = 16 * TT, TPWV = TPB / NW, NP = NOISY ? 2 : 1;
    __shared__ floatx4 s_part[NP][NW][TT][64];
    __shared__ int s_cnt[64];
    __shared__ float s_P[NW][64];
    __shared__ float s_H[NW];
    // per wave: the block's 16 * TT token rows x 128 columns of x, 16 slots of 16 bytes per row, slot
    // j of row R at position j ^ (R % 16)
    constexpr int XI = TPB / 4;  // load instructions per 128-column step: 4 rows of 256 bytes each
    __shared__ u32x4 s_x[NW][TPB * 16];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    if (blockIdx.x == 0 && threadIdx.x == 0) *ticket = 0;  // for a route_finalize_kernel that follows
    if (threadIdx.x < 64) s_cnt[threadIdx.x] = 0;
    const int64_t t0 = (int64_t)blockIdx.x * TPB;
    const int r = lane & 15, g = lane >> 4;
    const uint16_t* xr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int64_t t = t0 + tt * 16 + r;
        xr[tt] = x + (t < T ? t : T - 1) * d;
    }
    // the 128-column steps read x as whole 256-byte row pieces: load q covers rows 4q + lane / 16,
    // lane % 16 taking the row's 16-byte slot lane % 16
    const uint16_t* xq[XI];
    int xw[XI];
#pragma unroll
    for (int q = 0; q < XI; ++q) {
        const int R = q * 4 + g;
        const int64_t t = t0 + R;
        xq[q] = x + (t < T ? t : T - 1) * d + r * 8;
        xw[q] = R * 16 + (r ^ (R & 15));
    }
    const bool w_ok = r < E;  // padded expert rows are zero and not loaded
    const int nc = d / 32;
    const int kb0 = (wave * nc / NW) * 32, kb1 = ((wave + 1) * nc / NW) * 32;
    const floatx4 fzero = {0.f, 0.f, 0.f, 0.f};
    u32x4 xv[2][XI];
    floatx4 wf[2][4][2];
    // hi / mid / lo bf16 terms of 8 fp32 weights
    auto split8 = [](const floatx4 (&v)[2], bf16x8& h8, bf16x8& m8, bf16x8& l8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float f = v[j >> 2][j & 3];
            const __bf16 h = (__bf16)f;
            const float r1 = f - (float)h;
            const __bf16 m = (__bf16)r1;
            const float r2 = r1 - (float)m;
            h8[j] = h;
            m8[j] = m;
            l8[j] = (__bf16)r2;
        }
    };
    // a step's router loads go out before its x loads, so (loads complete in order) the split of the
    // router into bf16 terms runs while x is still arriving
#define RF_LOAD(b_, kb_)                                                                                  \
    {                                                                                                     \
        const int base = (kb_) + g * 8;                                                                   \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                   \
            wf[b_][i][0] = w_ok ? *reinterpret_cast<const floatx4*>(wr + base + i * 32) : fzero;          \
            wf[b_][i][1] = w_ok ? *reinterpret_cast<const floatx4*>(wr + base + i * 32 + 4) : fzero;      \
        }                                                                                                 \
        _Pragma("unroll") for (int q = 0; q < XI; ++q) xv[b_][q] = x_load(xq[q] + (kb_));                 \
    }
#define RF_MMA(b_)                                                                                        \
    {                                                                                                     \
        bf16x8 w3[4][3];                                                                                  \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) split8(wf[b_][i], w3[i][0], w3[i][1], w3[i][2]);    \
        __builtin_amdgcn_wave_barrier();                                                                  \
        _Pragma("unroll") for (int q = 0; q < XI; ++q) s_x[wave][xw[q]] = xv[b_][q];                      \
        __builtin_amdgcn_wave_barrier();                                                                  \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                                   \
            _Pragma("unroll") for (int tt = 0; tt < TT; ++tt) {                                           \
                const bf16x8 a_ = __builtin_bit_cast(bf16x8, s_x[wave][(tt * 16 + r) * 16 + ((4 * i + g) ^ r)]); \
                _Pragma("unroll") for (int p = 0; p < 3; ++p)                                             \
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_, w3[i][p], acc[tt], 0, 0, 0);    \
            }                                                                                             \
        }                                                                                                 \
    }
    // x is read once per pass; with a second pass it is loaded normally so that it stays in L2
    auto x_load = [](const uint16_t* p_) {
        return NOISY ? *reinterpret_cast<const u32x4*>(p_)
                     : __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p_));
    };
    for (int pass = 0; pass < NP; ++pass) {
    const float* wr = (pass == 0 ? w : w_noise) + (int64_t)(w_ok ? r : 0) * d;
    floatx4 acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
    int kb = kb0;
    const int nsteps = (kb1 - kb0) / 128;
    if (nsteps > 0) {
        RF_LOAD(0, kb)
        int st = 0;
        for (; st + 2 <= nsteps; st += 2) {
            if (st + 1 < nsteps) RF_LOAD(1, kb + 128)
            RF_MMA(0)
            if (st + 2 < nsteps) RF_LOAD(0, kb + 256)
            RF_MMA(1)
            kb += 256;
        }
        if (st < nsteps) {
            RF_MMA(0)
            kb += 128;
        }
    }
#undef RF_LOAD
#undef RF_MMA
    for (; kb < kb1; kb += 32) {  // 32-wide tail of the wave's range
        const int base = kb + g * 8;
        floatx4 w8[2] = {w_ok ? *reinterpret_cast<const floatx4*>(wr + base) : fzero,
                         w_ok ? *reinterpret_cast<const floatx4*>(wr + base + 4) : fzero};
        bf16x8 w3[3];
        split8(w8, w3[0], w3[1], w3[2]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(xr[tt] + base));
#pragma unroll
            for (int p = 0; p < 3; ++p) acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w3[p], acc[tt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) s_part[pass][wave][tt][lane] = acc[tt];
    }  // pass
    __syncthreads();
    // Selection, one token per 16-lane DPP row: wave w takes tokens 4w + r (r = lane / 16) of the
    // block, lane e = lane % 16 of a row holds expert e. The same steps as select_token, with the
    // wave reductions replaced by row reductions, so a wave selects its tokens together.
    const float* sp = reinterpret_cast<const float*>(&s_part[0][0][0][0]);
    const bool softmax = score == MOE_SOFTMAX;
    const int row = lane >> 4, e = lane & 15;
    const int lt = wave * TPWV + row;
    const int64_t t = t0 + lt;
    const bool valid = row < TPWV && t < T;
    const bool live = valid && e < E;
    // the 16x16 accumulator of token tile tt: lane c holds column (expert) c % 16 and rows (tokens)
    // 4 (c / 16) + v; the eight wave partials are summed in wave order
    float l = -INFINITY;
    if (live) {
        const int tt = lt >> 4, r16 = lt & 15;
        const int off = (tt * 64 + e + 16 * (r16 >> 2)) * 4 + (r16 & 3);
        float sum = sp[off];
#pragma unroll
        for (int wv = 1; wv < NW; ++wv) sum += sp[wv * TT * 256 + off];
        l = sum;
        if (NOISY) {  // the noise-scale logit, summed the same way
            const float* sq = sp + NW * TT * 256;
            float sn = sq[off];
#pragma unroll
            for (int wv = 1; wv < NW; ++wv) sn += sq[wv * TT * 256 + off];
            l = l + noise[t * E + e] * softplusf_(sn);
        }
        if (logits_out != nullptr) logits_out[t * E + e] = l;
    }
    const float m = row_max(l);
    const float p = live ? (softmax ? expf(l - m) : sigmoidf_(l)) : 0.f;
    const float Z = row_sum(p);
    const float invZ = 1.0f / Z, lnZ = logf(Z);
    const float pn = live ? p * invZ : 0.f;
    float hcur = 0.f;
    if (pn > 0.f) hcur = -pn * (softmax ? (l - m) - lnZ : logf(pn));
    float kv = softmax ? l : p;  // p holds the raw sigmoid score here
    kv = kv + (live && sel_bias != nullptr ? sel_bias[e] : 0.f);
    kv = kv + 0.0f;  // -0 -> +0: equal keys compare equal
    uint64_t key = live ? pack_key(kv, e) : 0ull;
    int sel_e = 0;
    for (int j = 0; j < k; ++j) {
        const uint64_t best = row_max_u64(key);
        const int ej = key_index(best);  // uniform over the row
        if (e == ej) key = 0ull;
        if (e == j) sel_e = ej;
    }
    // unbiased logit of slot j's expert, fetched from that expert's lane of the row
    const float sel_l = __shfl(l, (lane & 48) + sel_e);
    const bool slot = valid && e < k;
    const float lv = slot ? sel_l : -INFINITY;
    float gate;
    if (softmax) {
        if (renorm) {
            const float ms = row_max(lv);
            const float ex = slot ? expf(lv - ms) : 0.f;
            gate = ex / row_sum(ex);
        } else {
            gate = expf(lv - m) * invZ;
        }
    } else {
        const float sg = slot ? sigmoidf_(lv) : 0.f;
        gate = sg / row_sum(sg);
    }
    if (slot) {
        topk_idx[t * k + e] = sel_e;
        topk_w[t * k + e] = gate;
        atomicAdd(&s_cnt[sel_e], 1);
    }
    // the wave's partials: per expert the sum over its tokens in row order; the entropy terms summed
    // the same way, then over the row
    const float p1 = __shfl(pn, lane + 16), p2 = __shfl(pn, lane + 32), p3 = __shfl(pn, lane + 48);
    const float h1 = __shfl(hcur, lane + 16), h2 = __shfl(hcur, lane + 32), h3 = __shfl(hcur, lane + 48);
    const float hw = row_sum(((hcur + h1) + h2) + h3);
    if (lane < E) s_P[wave][lane] = ((pn + p1) + p2) + p3;
    if (lane == 0) s_H[wave] = hw;
    __syncthreads();
    if (threadIdx.x < E) {
        const int ex = threadIdx.x;
        blk_counts[(int64_t)blockIdx.x * E + ex] = s_cnt[ex];
        if (blk_P != nullptr) {
            float sp2 = s_P[0][ex];
#pragma unroll
            for (int wv = 1; wv < NW; ++wv) sp2 += s_P[wv][ex];
            blk_P[(int64_t)blockIdx.x * E + ex] = sp2;
        }
    }
    if (threadIdx.x == 0 && blk_H != nullptr) {
        float sh = s_H[0];
#pragma unroll
        for (int wv = 1; wv < NW; ++wv) sh += s_H[wv];
        blk_H[blockIdx.x] = sh;
    }
}

bool route_small_ok(int dtype, int E, int k, int d) {
    return dtype == MOE_BF16 && E <= 16 && k <= E && d % 32 == 0;
}

int route_small_tokens_per_block(int64_t T, int E, bool noisy) {
    (void)E;
    // two token tiles per block still leave a block per CU; the noisy kernel keeps one tile (a second
    // one would spill registers with both projections' loop state live)
    return !noisy && T >= 32 * 256 ? 32 : 16;
}

void launch_route_small(const void* x, const float* w_router, const float* w_noise, const float* noise,
                        const float* sel_bias, int64_t T, int d, int E, int k, int score, int renorm, float* logits,
                        int32_t* topk_idx, float* topk_w, int32_t* blk_counts, float* blk_P, float* blk_H,
                        int32_t* ticket, hipStream_t s) {
    const bool noisy = w_noise != nullptr;
    const int tpb = route_small_tokens_per_block(T, E, noisy);
    const unsigned nblk = (unsigned)((T + tpb - 1) / tpb);
    const auto xb = static_cast<const uint16_t*>(x);
#define MOE_ROUTE_FUSED(TT_, NOISY_)                                                                      \
    route_fused_kernel<TT_, NOISY_><<<nblk, kFusedRouteWaves * 64, 0, s>>>(                               \
        xb, w_router, w_noise, noise, sel_bias, T, d, E, k, score, renorm, logits, topk_idx, topk_w, blk_counts, \
        blk_P, blk_H, ticket)
    if (noisy) MOE_ROUTE_FUSED(1, true);
    else if (tpb == 32) MOE_ROUTE_FUSED(2, false);
    else MOE_ROUTE_FUSED(1, false);
#undef MOE_ROUTE_FUSED
}

// Expert counts and balance statistics from the per-block partials, in fixed-order sums (float64
// for the statistics): block e < E reduces expert e (count; with stats, f = counts/T and P = mean
// p), block E the entropy; the last block to finish (ticket) forms aux = E * sum_e f_e P_e over the
// per-expert products in a fixed order.
__global__ __launch_bounds__(256) void route_finalize_kernel(const int32_t* __restrict__ blk_counts,
                                                             const float* __restrict__ blk_P,
                                                             const float* __restrict__ blk_H, int nblk,
                                                             int64_t T, int E, int32_t* __restrict__ counts,
                                                             double* __restrict__ fp_scratch,
                                                             int32_t* __restrict__ ticket,
                                                             float* __restrict__ stats) {
    __shared__ double s_sum[256];
    __shared__ int s_cnt[256];
    __shared__ bool s_last;
    const int tid = threadIdx.x;
    const int e = blockIdx.x;
    const double invT = 1.0 / (double)T;
    double acc = 0.0;
    int cnt = 0;
    if (e < E) {
        for (int b = tid; b < nblk; b += 256) {
            cnt += blk_counts[(int64_t)b * E + e];
            if (stats) acc += (double)blk_P[(int64_t)b * E + e];
        }
    } else if (stats) {
        for (int b = tid; b < nblk; b += 256) acc += (double)blk_H[b];
    }
    s_sum[tid] = acc;
    s_cnt[tid] = cnt;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            s_sum[tid] += s_sum[tid + o];
            s_cnt[tid] += s_cnt[tid + o];
        }
        __syncthreads();
    }
    if (tid == 0 && e < E) counts[e] = s_cnt[0];
    if (stats == nullptr) return;
    if (tid == 0) {
        if (e < E) {
            const double f = (double)s_cnt[0] * invT, Pm = s_sum[0] * invT;
            stats[e] = (float)f;
            stats[E + e] = (float)Pm;
            fp_scratch[e] = f * Pm;
        } else {
            stats[2 * E + 1] = (float)(s_sum[0] * invT);
        }
        __threadfence();
        s_last = atomicAdd(ticket, 1) == (int)gridDim.x - 1;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // sum_e f_e P_e: each thread sums experts tid, tid + 256, ... in order, then a fixed tree
    double a = 0.0;
    for (int i = tid; i < E; i += 256) a += __builtin_nontemporal_load(fp_scratch + i);
    s_sum[tid] = a;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) s_sum[tid] += s_sum[tid + o];
        __syncthreads();
    }
    if (tid == 0) {
        stats[2 * E] = (float)((double)E * s_sum[0]);
        *ticket = 0;  // left at zero for the next call (every block has taken its ticket)
    }
}

// Aux-loss-free balancing step ("Router Optimization Techniques", How It Works 2 and Fine-Tuning
// Strategies 1): sel_bias[e] -= gamma * sign(counts[e] - T*k/E), the sign taken exactly in
// integers and the step as one fp32 subtraction.
__global__ __launch_bounds__(256) void route_bias_update_kernel(const int32_t* __restrict__ counts, int64_t T,
                                                                int E, int k, float gamma,
                                                                float* __restrict__ sel_bias) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    const int64_t diff = (int64_t)counts[e] * E - T * k;
    const float step = diff > 0 ? gamma : (diff < 0 ? -gamma : 0.0f);
    sel_bias[e] = sel_bias[e] - step;
}

void launch_route_bias_update(const int32_t* counts, int64_t T, int E, int k, float gamma, float* sel_bias,
                              hipStream_t s) {
    route_bias_update_kernel<<<(unsigned)((E + 255) / 256), 256, 0, s>>>(counts, T, E, k, gamma, sel_bias);
}

void launch_route_prep(const float* w_router, int E, int Epad, int d, uint16_t* wsplit, int32_t* ticket,
                       hipStream_t s) {
    const int64_t n = wsplit ? (int64_t)Epad * d : 0;
    const unsigned grid = (unsigned)(n > 0 ? (n / 4 + 255) / 256 : 1);
    route_prep_kernel<<<grid, 256, 0, s>>>(w_router, E, Epad, d, wsplit, ticket);
}

void launch_route_logits(int dtype, const void* x, const float* w_router, const uint16_t* wsplit, int Epad,
                         float* logits, int64_t T, int d, int E, hipStream_t s) {
    if (dtype == MOE_BF16) {
        const auto xb = static_cast<const uint16_t*>(x);
        const bool nt = Epad == 16;
        // one 16-expert tile: eight waves split d, more loads in flight per token tile
        if (nt && T >= 32 * 256) {
            dim3 grid((unsigned)((T + 31) / 32), 1);
            route_logits_bf16_kernel<2, true, 8><<<grid, 512, 0, s>>>(xb, wsplit, Epad, logits, T, d, E);
        } else if (nt) {
            dim3 grid((unsigned)((T + 15) / 16), 1);
            route_logits_bf16_kernel<1, true, 8><<<grid, 512, 0, s>>>(xb, wsplit, Epad, logits, T, d, E);
        } else if (T >= 32 * 256) {  // two token tiles per wave still leave a block per CU
            dim3 grid((unsigned)((T + 31) / 32), (unsigned)(Epad / 16));
            route_logits_bf16_kernel<2, false, 4><<<grid, 256, 0, s>>>(xb, wsplit, Epad, logits, T, d, E);
        } else {
            dim3 grid((unsigned)((T + 15) / 16), (unsigned)(Epad / 16));
            route_logits_bf16_kernel<1, false, 4><<<grid, 256, 0, s>>>(xb, wsplit, Epad, logits, T, d, E);
        }
    } else {
        const int64_t n = T * E;
        route_logits_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<const float*>(x),
                                                                           w_router, logits, T, d, E);
    }
}

// route_select_kernel for wide routers (16 < E <= 16 * EPR, k <= 16) with one token per 16-lane DPP
// row: four tokens per wave, four waves per block (the same 16-token blocks and partials). Lane c of a
// row holds experts c + 16 i, so each logit load reads 64 contiguous bytes per row. The steps are
// select_token's, with the wave reductions replaced by row reductions (route_fused_kernel's
// selection with EPR experts per lane); the wave's per-expert partials add its four rows in order.
constexpr int64_t kSelRowsMinTokens = 8192;
template <int EPR>
__global__ __launch_bounds__(256) void route_select_rows_kernel(
    const float* __restrict__ logits, int lg_ld, int lg_split, float* __restrict__ logits_out,
    const float* __restrict__ sel_bias, int64_t T, int E, int k, int score, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ blk_counts, float* __restrict__ blk_P, float* __restrict__ blk_H,
    const float* __restrict__ s_logits, const float* __restrict__ noise, float* __restrict__ h_out) {
    constexpr int NWV = kRouteTokensPerBlock / 4;
    __shared__ int s_cnt[16 * EPR];
    __shared__ float s_P[NWV][16 * EPR];
    __shared__ float s_H[NWV];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int row = lane >> 4, c = lane & 15;
    for (int e = threadIdx.x; e < 16 * EPR; e += NWV * 64) s_cnt[e] = 0;
    __syncthreads();
    const bool softmax = score == MOE_SOFTMAX;
    const int64_t t = (int64_t)blockIdx.x * kRouteTokensPerBlock + wave * 4 + row;
    const bool valid = t < T;
    auto logit_at = [&](const float* lg, int e) {
        const float* r = lg + t * lg_ld + e;
        return lg_split > 0 ? (r[0] + r[lg_split]) + r[2 * lg_split] : r[0];
    };
    float l[EPR];
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
        const int e = c + 16 * i;
        l[i] = valid && e < E ? logit_at(logits, e) : -INFINITY;
    }
    if (s_logits != nullptr) {
#pragma unroll
        for (int i = 0; i < EPR; ++i) {
            const int e = c + 16 * i;
            if (valid && e < E) {
                const int64_t o = t * E + e;
                l[i] = l[i] + noise[o] * softplusf_(logit_at(s_logits, e));
                if (h_out != nullptr) h_out[o] = l[i];
            }
        }
    } else if (logits_out != nullptr) {
#pragma unroll
        for (int i = 0; i < EPR; ++i) {
            const int e = c + 16 * i;
            if (valid && e < E) logits_out[t * E + e] = l[i];
        }
    }
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPR; ++i) lm = fmaxf(lm, l[i]);
    const float m = row_max(lm);
    // distribution whose mean is P_e and whose entropy is reported
    float p[EPR];
    float zpart = 0.f;
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
        const bool live = valid && c + 16 * i < E;
        p[i] = live ? (softmax ? expf(l[i] - m) : sigmoidf_(l[i])) : 0.f;
        zpart += p[i];
    }
    const float Z = row_sum(zpart);
    const float invZ = 1.0f / Z, lnZ = logf(Z);
    uint64_t key[EPR];
    float pn[EPR];
    float hpart = 0.f;
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
        const int e = c + 16 * i;
        const bool live = valid && e < E;
        pn[i] = live ? p[i] * invZ : 0.f;
        if (pn[i] > 0.f) hpart -= pn[i] * (softmax ? (l[i] - m) - lnZ : logf(pn[i]));
        float kv = softmax ? l[i] : p[i];  // p[i] holds the raw sigmoid score here
        kv = kv + (live && sel_bias != nullptr ? sel_bias[e] : 0.f);
        kv = kv + 0.0f;  // -0 -> +0: equal keys compare equal
        key[i] = live ? pack_key(kv, e) : 0ull;
    }
    int sel_e = 0;
    float sel_l = -INFINITY;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < EPR; ++i) best = key[i] > best ? key[i] : best;
        best = row_max_u64(best);
        const int ej = key_index(best);  // uniform over the row
        // unbiased logit of the winner, read from the lane of the row that holds it
        float mine = 0.f;
#pragma unroll
        for (int i = 0; i < EPR; ++i) {
            if ((ej >> 4) == i) mine = l[i];
            if (ej == c + 16 * i) key[i] = 0ull;
        }
        const float le = __shfl(mine, (lane & 48) + (ej & 15));
        if (c == j) {
            sel_e = ej;
            sel_l = le;
        }
    }
    // gates from the unbiased logits of the selection (lane j of the row holds slot j)
    const bool slot = valid && c < k;
    const float lv = slot ? sel_l : -INFINITY;
    float gate;
    if (softmax) {
        if (renorm) {
            const float ms = row_max(lv);
            const float ex = slot ? expf(lv - ms) : 0.f;
            gate = ex / row_sum(ex);
        } else {
            gate = expf(lv - m) * invZ;
        }
    } else {
        const float sg = slot ? sigmoidf_(lv) : 0.f;
        gate = sg / row_sum(sg);
    }
    if (slot) {
        topk_idx[t * k + c] = sel_e;
        topk_w[t * k + c] = gate;
        atomicAdd(&s_cnt[sel_e], 1);
    }
    // the wave's partials: per expert its four tokens in row order; the entropy terms the same way,
    // then over the row
#pragma unroll
    for (int i = 0; i < EPR; ++i) {
        const float p1 = __shfl(pn[i], lane + 16), p2 = __shfl(pn[i], lane + 32), p3 = __shfl(pn[i], lane + 48);
        const int e = c + 16 * i;
        if (lane < 16 && e < E) s_P[wave][e] = ((pn[i] + p1) + p2) + p3;
    }
    const float h1 = __shfl(hpart, lane + 16), h2 = __shfl(hpart, lane + 32), h3 = __shfl(hpart, lane + 48);
    const float hw = row_sum(((hpart + h1) + h2) + h3);
    if (lane == 0) s_H[wave] = hw;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += NWV * 64) {
        blk_counts[(int64_t)blockIdx.x * E + e] = s_cnt[e];
        if (blk_P != nullptr) {
            float sp = s_P[0][e];
#pragma unroll
            for (int w = 1; w < NWV; ++w) sp += s_P[w][e];
            blk_P[(int64_t)blockIdx.x * E + e] = sp;
        }
    }
    if (threadIdx.x == 0 && blk_H != nullptr) {
        float sh = s_H[0];
#pragma unroll
        for (int w = 1; w < NWV; ++w) sh += s_H[w];
        blk_H[blockIdx.x] = sh;
    }
}

void launch_route_select(const float* logits, int lg_ld, int lg_split, float* logits_out, const float* sel_bias,
                         int64_t T, int E, int k, int score, int renorm, int32_t* topk_idx, float* topk_w,
                         int32_t* blk_counts, float* blk_P, float* blk_H, const float* s_logits, const float* noise,
                         float* h_out, hipStream_t s) {
    const unsigned nblk = (unsigned)((T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock);
    // four tokens per wave pays once the batch still fills the chip with waves (measured: Qwen3-shaped
    // T = 16384, E = 128: 91.6 against 98.7 us for the route; DeepSeek-shaped T = 4096, E = 256: 108
    // against 104 us)
    if (E > 16 && E <= 256 && k <= 16 && T >= kSelRowsMinTokens) {
#define MOE_SELECT_ROWS(EPR)                                                                             \
    route_select_rows_kernel<EPR><<<nblk, 256, 0, s>>>(logits, lg_ld, lg_split, logits_out, sel_bias, T, E, k, score, \
                                                       renorm, topk_idx, topk_w, blk_counts, blk_P, blk_H, s_logits, \
                                                       noise, h_out)
        if (E <= 32) MOE_SELECT_ROWS(2);
        else if (E <= 64) MOE_SELECT_ROWS(4);
        else if (E <= 128) MOE_SELECT_ROWS(8);
        else MOE_SELECT_ROWS(16);
#undef MOE_SELECT_ROWS
        return;
    }
#define MOE_SELECT(EPL)                                                                                  \
    route_select_kernel<EPL><<<nblk, kSelWaves * 64, 0, s>>>(logits, lg_ld, lg_split, logits_out, sel_bias, T, E, k, score, \
                                                 renorm, topk_idx, topk_w, blk_counts, blk_P, blk_H, s_logits, \
                                                 noise, h_out)
    if (E <= 64) MOE_SELECT(1);
    else if (E <= 128) MOE_SELECT(2);
    else if (E <= 256) MOE_SELECT(4);
    else if (E <= 512) MOE_SELECT(8);
    else MOE_SELECT(16);
#undef MOE_SELECT
}

void launch_route_finalize(const int32_t* blk_counts, const float* blk_P, const float* blk_H, int nblk, int64_t T,
                           int E, int32_t* counts, double* fp_scratch, int32_t* ticket, float* stats,
                           hipStream_t s) {
    if (E <= kFinalizeSmallExperts) {
        route_finalize_small_kernel<<<1, 1024, 0, s>>>(blk_counts, blk_P, blk_H, nblk, T, E, counts, stats);
        return;
    }
    route_finalize_kernel<<<(unsigned)(stats ? E + 1 : E), 256, 0, s>>>(blk_counts, blk_P, blk_H, nblk, T, E,
                                                                         counts, fp_scratch, ticket, stats);
}

}  // namespace moe

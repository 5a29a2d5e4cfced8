// libmoe C ABI (include/moe.h): argument validation, workspace planning and stage launches.
// Every check runs before the first HIP call, so a rejected call enqueues nothing and the
// validation paths run on hosts without a GPU.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/moe.h"
#include "moe_kernels.h"

namespace {

using moe::kPermTile;
using moe::kRouteTokensPerBlock;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_shape(const moe_shape* s) {
    if (s == nullptr) return MOE_ERR_INVALID_ARG;
    if (s->T < 0 || s->E < 1 || s->E > 1024 || s->k < 1 || s->k > s->E || s->k > 32) return MOE_ERR_INVALID_ARG;
    if (s->d_model <= 0 || s->d_ff <= 0 || s->d_ff_shared < 0) return MOE_ERR_INVALID_ARG;
    if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (s->act != MOE_GELU_MLP && s->act != MOE_SWIGLU) return MOE_ERR_INVALID_ARG;
    if (s->score != MOE_SOFTMAX && s->score != MOE_SIGMOID) return MOE_ERR_INVALID_ARG;
    if (s->renorm != 0 && s->renorm != 1) return MOE_ERR_INVALID_ARG;
    if (s->capacity < 0) return MOE_ERR_INVALID_ARG;
    if (s->T * (int64_t)s->k > (int64_t)INT32_MAX) return MOE_ERR_INVALID_ARG;
    if (s->score == MOE_SIGMOID && s->renorm != 1) return MOE_ERR_UNSUPPORTED;
    // 16-byte vectors of bf16 (8 elements) or fp32 (4 elements) along every row
    const int mult = s->dtype == MOE_BF16 ? 8 : 4;
    if (s->d_model % mult || s->d_ff % mult || s->d_ff_shared % mult) return MOE_ERR_INVALID_ARG;
    // the GEMM kernels' DMA offsets are 32-bit: at most 640 operand rows of K bf16 elements per tile,
    // with K up to 2 * d_ff (the backward's products against the transposed gate/up weights)
    if (s->d_model > MOE_MAX_WIDTH || s->d_ff > MOE_MAX_WIDTH || s->d_ff_shared > MOE_MAX_WIDTH)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

inline int elem_bytes(const moe_shape* s) { return s->dtype == MOE_BF16 ? 2 : 4; }

// ---- workspace layouts (each region 256-byte aligned) ----------------------------------------
struct Carver {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    }
};

struct RouteWs {
    size_t logits, wsplit, blk_counts, blk_P, blk_H, fp, ticket, gpart, bytes;
    int nblk, Epad;
    bool gemm;  // logits as a dense product of x and the split router through the grouped GEMM
    int lg_ld, lg_split;
};
RouteWs route_ws(const moe_shape* s) {
    RouteWs w;
    Carver c;
    w.nblk = (int)cdiv(s->T, kRouteTokensPerBlock);
    w.Epad = (int)cdiv(s->E, 16) * 16;
    // the MFMA logits kernels step d in 32-column chunks; other widths take the router product on the
    // grouped GEMM, whose last K stage is masked
    w.gemm = s->dtype == MOE_BF16 && (w.Epad >= moe::kRouteGemmMinEpad || s->d_model % 32 != 0);
    w.lg_ld = w.gemm ? 3 * w.Epad : s->E;
    w.lg_split = w.gemm ? w.Epad : 0;
    w.logits = c.take((size_t)s->T * w.lg_ld * 4);
    w.wsplit = c.take(s->dtype == MOE_BF16 ? (size_t)3 * w.Epad * s->d_model * 2 : 0);
    w.blk_counts = c.take((size_t)w.nblk * s->E * 4);
    w.blk_P = c.take((size_t)w.nblk * s->E * 4);
    w.blk_H = c.take((size_t)w.nblk * 4);
    w.fp = c.take((size_t)s->E * 8);
    w.ticket = c.take(4);
    w.gpart = c.take(w.gemm ? moe::gemm_partials_bytes(s->dtype) : 0);
    w.bytes = c.off;
    return w;
}

// noisy routing: the route workspace plus the noise projection's logits and split
struct RouteNoisyWs {
    RouteWs base;
    size_t s_logits, wsplit_n, bytes;
};
RouteNoisyWs route_noisy_ws(const moe_shape* s) {
    RouteNoisyWs w;
    w.base = route_ws(s);
    Carver c;
    c.off = w.base.bytes;
    w.s_logits = c.take((size_t)s->T * w.base.lg_ld * 4);
    w.wsplit_n = c.take(s->dtype == MOE_BF16 ? (size_t)3 * w.base.Epad * s->d_model * 2 : 0);
    w.bytes = c.off;
    return w;
}

struct PermWs {
    size_t tile_counts, tile_base, bytes;
    int ntiles;
};
PermWs perm_ws(const moe_shape* s) {
    PermWs w;
    Carver c;
    w.ntiles = (int)cdiv(s->T * s->k, kPermTile);
    w.tile_counts = c.take((size_t)w.ntiles * s->E * 4);
    w.tile_base = c.take((size_t)w.ntiles * s->E * 4);
    w.bytes = c.off;
    return w;
}

// fp32 partial tiles of the grouped GEMM's split last round (bf16 layers only)
struct ExpertWs {
    size_t partials, bytes;
};
ExpertWs expert_ws(const moe_shape* s) {
    ExpertWs w;
    Carver c;
    w.partials = c.take(moe::gemm_partials_bytes(s->dtype));
    w.bytes = c.off;
    return w;
}

struct FfnWs {
    size_t h, partials, bytes;
};
FfnWs ffn_ws(const moe_shape* s) {
    FfnWs w;
    Carver c;
    w.h = c.take((size_t)s->T * s->k * s->d_ff * elem_bytes(s));
    w.partials = c.take(moe::gemm_partials_bytes(s->dtype));
    w.bytes = c.off;
    return w;
}

struct SharedWs {
    size_t hs, partials, bytes;
};
SharedWs shared_ws(const moe_shape* s) {
    SharedWs w;
    Carver c;
    w.hs = c.take((size_t)s->T * s->d_ff_shared * elem_bytes(s));
    w.partials = c.take(s->d_ff_shared ? moe::gemm_partials_bytes(s->dtype) : 0);
    w.bytes = c.off;
    return w;
}

// bf16 forward: the up projection reads token rows through sorted_token (no x_perm copy) while x
// stays below 2 GB, so that the offset the kernels give rows past a group's end lies out of range
bool fwd_gathers(const moe_shape* s) {
    return s->dtype == MOE_BF16 && s->T * (int64_t)s->d_model * 2 < ((int64_t)1 << 31);
}

struct FwdWs {
    size_t topk_idx, topk_w, counts, offsets, sorted_token, inv_pos, x_perm, y_perm, ys, scratch, bytes;
};
FwdWs fwd_ws(const moe_shape* s) {
    FwdWs w;
    Carver c;
    const size_t A = (size_t)s->T * s->k, eb = elem_bytes(s);
    w.topk_idx = c.take(A * 4);
    w.topk_w = c.take(A * 4);
    w.counts = c.take((size_t)s->E * 4);
    w.offsets = c.take((size_t)(s->E + 1) * 4);
    // the gathering GEMM reads sorted_token 16 rows at a time from a group's tile start, up to 255
    // entries past the last row
    w.sorted_token = c.take((A + 256) * 4);
    w.inv_pos = c.take(A * 4);
    w.x_perm = c.take(fwd_gathers(s) ? 0 : A * s->d_model * eb);
    w.y_perm = c.take(A * s->d_model * eb);
    w.ys = c.take(s->d_ff_shared ? (size_t)s->T * s->d_model * eb : 0);
    size_t scratch = route_ws(s).bytes;  // the stages run one after another on one stream
    if (perm_ws(s).bytes > scratch) scratch = perm_ws(s).bytes;
    if (ffn_ws(s).bytes > scratch) scratch = ffn_ws(s).bytes;
    if (s->d_ff_shared && shared_ws(s).bytes > scratch) scratch = shared_ws(s).bytes;
    w.scratch = c.take(scratch);
    w.bytes = c.off;
    return w;
}

// backward: intermediates of the chain rule (rows = T*k bound of the permuted buffer)
// bf16 layers with many rows per expert run the two dgrad products on the persistent GEMM against
// transposed copies of the expert weights (the strided GEMM otherwise). Transposing costs four bytes
// of traffic per weight byte; the faster products save time in proportion to the rows per expert.
// Measured: +8 % at 2048 rows per expert (Mixtral-shaped), even at 1024 (Qwen3-shaped), a loss at 128
// (DeepSeek-shaped, 22.5 GB of weights).
constexpr int64_t kBwdTransposedMinRows = 1536;
bool bwd_dgrad_transposed(const moe_shape* s) {
    return s->dtype == MOE_BF16 && s->T * s->k >= kBwdTransposedMinRows * s->E;
}
// The same layers run the two weight gradients on the wide GEMM's K-grouped mode, from transposed,
// per-expert zero-padded copies of the permuted buffers (their output rows d and n_in must be
// multiples of 256, the transposed widths multiples of 64); the strided GEMM otherwise.
// columns of the transposed copies: every expert's rows padded to a multiple of 64, at least 64
int64_t bwd_wgrad_ld(const moe_shape* s) { return (s->T * s->k + 63) / 64 * 64 + 64 * (int64_t)s->E; }
// The K-grouped product's DMA offsets are 32-bit: a tile's 256 + 384 operand rows of ld bf16
// elements must stay below 2^31 bytes. Longer token batches take the strided GEMM (64-bit addresses).
constexpr int64_t kKgMaxLd = (((int64_t)1 << 31) - 1) / ((256 + 384) * 2);
bool bwd_wgrad_kgrouped(const moe_shape* s) {
    const int64_t n_in = s->act == MOE_SWIGLU ? 2 * (int64_t)s->d_ff : s->d_ff;
    return bwd_dgrad_transposed(s) && s->d_model % 256 == 0 && n_in % 256 == 0 && s->d_ff % 64 == 0 &&
           bwd_wgrad_ld(s) <= kKgMaxLd;
}

struct BwdWs {
    size_t dg, dYp, pre, h, dh, dAU, dXp, dx32, dl, partials, rpart, pre_s, hs, dhs, dAUs, dXs, w_inT, w_outT, wT1,
        wT2, poff, pblk, bytes;
};
BwdWs bwd_ws(const moe_shape* s) {
    BwdWs w;
    Carver c;
    const size_t A = (size_t)s->T * s->k, eb = elem_bytes(s), T = (size_t)s->T;
    const size_t d = s->d_model, F = s->d_ff, n_in = s->act == MOE_SWIGLU ? 2 * F : F, Fs = s->d_ff_shared;
    w.dg = c.take(A * 4);
    w.dYp = c.take(A * d * eb);
    w.pre = c.take(A * n_in * eb);
    w.h = c.take(A * F * eb);
    w.dh = c.take(A * F * 4);
    w.dAU = c.take(A * n_in * eb);
    w.dXp = c.take(A * d * 4);
    w.dx32 = c.take(T * d * 4);
    w.dl = c.take(T * s->E * 4);
    w.partials = c.take(moe::gemm_partials_bytes(s->dtype));
    w.rpart = c.take(moe::bwd_router_partials_bytes(s->T, s->E, s->d_model));
    w.pre_s = c.take(T * 2 * Fs * eb);
    w.hs = c.take(T * Fs * eb);
    w.dhs = c.take(T * Fs * 4);
    w.dAUs = c.take(T * 2 * Fs * eb);
    w.dXs = c.take(Fs ? T * d * 4 : 0);
    const bool tr = bwd_dgrad_transposed(s);
    w.w_inT = c.take(tr ? (size_t)s->E * n_in * d * 2 : 0);
    w.w_outT = c.take(tr ? (size_t)s->E * d * F * 2 : 0);
    const bool kg = bwd_wgrad_kgrouped(s);
    const size_t ld = kg ? (size_t)bwd_wgrad_ld(s) : 0;
    w.wT1 = c.take(kg ? (d > n_in ? d : n_in) * ld * 2 : 0);  // dY^T, then dAU^T
    w.wT2 = c.take(kg ? (F > d ? F : d) * ld * 2 : 0);        // h^T, then x_perm^T
    w.poff = c.take(kg ? ((size_t)s->E + 1) * 4 : 0);
    w.pblk = c.take(kg ? ld / 64 * 4 : 0);
    w.bytes = c.off;
    return w;
}

template <typename T>
inline T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

inline int launched() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ---- stage bodies (arguments already validated) ------------------------------------------------
// logits (fp32) of x and the router; bf16 layers split the router into hi/mid/lo first. With a wide
// router (w.gemm) lg receives the three products side by side ([T, 3 Epad]).
void route_logits(const moe_shape* s, const RouteWs& w, const void* x, const float* w_router, uint16_t* wsplit,
                  int32_t* ticket, float* lg, void* ws, hipStream_t st) {
    moe::launch_route_prep(w_router, s->E, w.Epad, s->d_model, wsplit, ticket, st);
    if (w.gemm)
        moe::launch_grouped_gemm(MOE_BF16, moe::EPI_F32, 128, x, wsplit, nullptr, lg, nullptr, 0, 1, 0, s->T, w.lg_ld,
                                 s->d_model, at<float>(ws, w.gpart), st);
    else
        moe::launch_route_logits(s->dtype, x, w_router, wsplit, w.Epad, lg, s->T, s->d_model, s->E, st);
}

void do_route(const moe_shape* s, const void* x, const float* w_router, const float* sel_bias, float* logits,
              int32_t* topk_idx, float* topk_w, int32_t* counts, float* stats, void* ws, hipStream_t st) {
    const RouteWs w = route_ws(s);
    float* lg = logits && !w.gemm ? logits : at<float>(ws, w.logits);
    uint16_t* wsplit = s->dtype == MOE_BF16 ? at<uint16_t>(ws, w.wsplit) : nullptr;
    int32_t* ticket = at<int32_t>(ws, w.ticket);
    int32_t* blk_counts = at<int32_t>(ws, w.blk_counts);
    float* blk_P = stats ? at<float>(ws, w.blk_P) : nullptr;
    float* blk_H = stats ? at<float>(ws, w.blk_H) : nullptr;
    if (moe::route_small_ok(s->dtype, s->E, s->k, s->d_model)) {  // logits and selection in one launch
        const int nblk = (int)cdiv(s->T, moe::route_small_tokens_per_block(s->T, s->E, false));
        moe::launch_route_small(x, w_router, nullptr, nullptr, sel_bias, s->T, s->d_model, s->E, s->k, s->score,
                                s->renorm, logits, topk_idx, topk_w, blk_counts, blk_P, blk_H, ticket, st);
        moe::launch_route_finalize(blk_counts, blk_P, blk_H, nblk, s->T, s->E, counts, at<double>(ws, w.fp), ticket,
                                   stats, st);
        return;
    }
    route_logits(s, w, x, w_router, wsplit, ticket, lg, ws, st);
    moe::launch_route_select(lg, w.lg_ld, w.lg_split, w.gemm ? logits : nullptr, sel_bias, s->T, s->E, s->k,
                             s->score, s->renorm, topk_idx, topk_w, blk_counts, blk_P, blk_H, nullptr, nullptr,
                             nullptr, st);
    moe::launch_route_finalize(blk_counts, blk_P, blk_H, w.nblk, s->T, s->E, counts, at<double>(ws, w.fp), ticket,
                               stats, st);
}

void do_route_noisy(const moe_shape* s, const void* x, const float* w_router, const float* w_noise,
                    const float* noise, const float* sel_bias, float* logits, int32_t* topk_idx, float* topk_w,
                    int32_t* counts, float* stats, void* ws, hipStream_t st) {
    const RouteNoisyWs wn = route_noisy_ws(s);
    const RouteWs& w = wn.base;
    float* lg = at<float>(ws, w.logits);
    float* sl = at<float>(ws, wn.s_logits);
    const bool bf = s->dtype == MOE_BF16;
    uint16_t* wsplit = bf ? at<uint16_t>(ws, w.wsplit) : nullptr;
    uint16_t* wsplit_n = bf ? at<uint16_t>(ws, wn.wsplit_n) : nullptr;
    int32_t* ticket = at<int32_t>(ws, w.ticket);
    int32_t* blk_counts = at<int32_t>(ws, w.blk_counts);
    float* blk_P = stats ? at<float>(ws, w.blk_P) : nullptr;
    float* blk_H = stats ? at<float>(ws, w.blk_H) : nullptr;
    if (moe::route_small_ok(s->dtype, s->E, s->k, s->d_model)) {  // both projections and the selection fused
        const int nblk = (int)cdiv(s->T, moe::route_small_tokens_per_block(s->T, s->E, true));
        moe::launch_route_small(x, w_router, w_noise, noise, sel_bias, s->T, s->d_model, s->E, s->k, s->score,
                                s->renorm, logits, topk_idx, topk_w, blk_counts, blk_P, blk_H, ticket, st);
        moe::launch_route_finalize(blk_counts, blk_P, blk_H, nblk, s->T, s->E, counts, at<double>(ws, w.fp), ticket,
                                   stats, st);
        return;
    }
    route_logits(s, w, x, w_router, wsplit, ticket, lg, ws, st);
    route_logits(s, w, x, w_noise, wsplit_n, ticket, sl, ws, st);
    moe::launch_route_select(lg, w.lg_ld, w.lg_split, nullptr, sel_bias, s->T, s->E, s->k, s->score, s->renorm,
                             topk_idx, topk_w, blk_counts, blk_P, blk_H, sl, noise, logits, st);
    moe::launch_route_finalize(blk_counts, blk_P, blk_H, w.nblk, s->T, s->E, counts, at<double>(ws, w.fp), ticket,
                               stats, st);
}

// x_perm == NULL: positions only (offsets, sorted_token, inv_pos), no row copy; the forward's up
// projection then reads the token rows through sorted_token itself
void do_permute(const moe_shape* s, const int32_t* topk_idx, const void* x, int32_t* offsets,
                int32_t* sorted_token, int32_t* inv_pos, void* x_perm, void* ws, hipStream_t st) {
    const PermWs w = perm_ws(s);
    const int64_t A = s->T * s->k;
    if (moe::perm_index_small_ok(A, s->E)) {
        moe::launch_perm_index_small(topk_idx, A, s->E, s->k, s->capacity, offsets, inv_pos, sorted_token, st);
        if (x_perm != nullptr) moe::launch_perm_scatter(x, inv_pos, s->T, s->d_model, s->k, elem_bytes(s), x_perm, st);
        return;
    }
    int32_t* tile_counts = at<int32_t>(ws, w.tile_counts);
    moe::launch_perm_local(topk_idx, A, s->E, tile_counts, inv_pos, st);  // inv_pos holds in-tile ranks
    int32_t* tile_base = nullptr;
    if (!moe::perm_fold_ok(A, s->E, s->k)) {
        tile_base = at<int32_t>(ws, w.tile_base);
        moe::launch_perm_scan(tile_counts, w.ntiles, A, s->E, s->capacity, tile_base, offsets, st);
    }
    moe::launch_perm_place_scatter(x, topk_idx, tile_counts, tile_base, offsets, s->E, s->capacity, s->T,
                                   s->d_model, s->k, x_perm != nullptr ? elem_bytes(s) : 0, inv_pos, sorted_token,
                                   x_perm, st);
}

inline float* partials_of(void* ws, size_t off, const moe_shape* s) {
    return s->dtype == MOE_BF16 ? at<float>(ws, off) : nullptr;
}

// gather != NULL: x_perm is the token matrix x and row p of the product reads x[gather[p]]
void do_up(const moe_shape* s, int e_begin, int e_end, const void* x_perm, const int32_t* offsets,
           const void* w_in, const void* b_in, void* h, float* partials, hipStream_t st,
           const int32_t* gather = nullptr) {
    const int64_t A = s->T * s->k;
    const moe::GemmPlan p = moe::plan_gemm(s->dtype, A / s->E, s->d_ff, s->d_model);
    moe::launch_grouped_gemm(s->dtype, s->act == MOE_SWIGLU ? moe::EPI_SWIGLU : moe::EPI_GELU_BIAS, p.bm, x_perm,
                             w_in, b_in, h, offsets, e_begin, e_end - e_begin, A, 0, s->d_ff, s->d_model, partials,
                             st, gather, s->T);
}

void do_down(const moe_shape* s, int e_begin, int e_end, const void* h, const int32_t* offsets, const void* w_out,
             const void* b_out, void* y_perm, float* partials, hipStream_t st) {
    const int64_t A = s->T * s->k;
    const moe::GemmPlan p = moe::plan_gemm(s->dtype, A / s->E, s->d_model, s->d_ff);
    moe::launch_grouped_gemm(s->dtype, moe::EPI_BIAS, p.bm, h, w_out, b_out, y_perm, offsets, e_begin,
                             e_end - e_begin, A, 0, s->d_model, s->d_ff, partials, st);
}

void do_ffn(const moe_shape* s, int e_begin, int e_end, const void* x_perm, const int32_t* offsets,
            const void* w_in, const void* b_in, const void* w_out, const void* b_out, void* y_perm, void* ws,
            hipStream_t st, const int32_t* gather = nullptr) {
    const FfnWs w = ffn_ws(s);
    void* h = at<void>(ws, w.h);
    float* partials = partials_of(ws, w.partials, s);
    // one up and one down launch over all experts: running them in chunks whose h fits the 256 MiB
    // last-level cache made the Mixtral-shaped step slower with the 256 x 384 tiles (4.79 against
    // 4.73 ms), so the down projection streams h from HBM
    do_up(s, e_begin, e_end, x_perm, offsets, w_in, b_in, h, partials, st, gather);
    do_down(s, e_begin, e_end, h, offsets, w_out, b_out, y_perm, partials, st);
}

void do_shared(const moe_shape* s, const void* x, const void* ws_in, const void* ws_out, void* y_shared, void* ws,
               hipStream_t st) {
    const SharedWs w = shared_ws(s);
    void* hs = at<void>(ws, w.hs);
    float* partials = partials_of(ws, w.partials, s);
    const moe::GemmPlan p1 = moe::plan_gemm(s->dtype, s->T, s->d_ff_shared, s->d_model);
    const moe::GemmPlan p2 = moe::plan_gemm(s->dtype, s->T, s->d_model, s->d_ff_shared);
    moe::launch_grouped_gemm(s->dtype, moe::EPI_SWIGLU, p1.bm, x, ws_in, nullptr, hs, nullptr, 0, 1, s->T, s->T,
                             s->d_ff_shared, s->d_model, partials, st);
    moe::launch_grouped_gemm(s->dtype, moe::EPI_BIAS, p2.bm, hs, ws_out, nullptr, y_shared, nullptr, 0, 1, s->T, s->T,
                             s->d_model, s->d_ff_shared, partials, st);
}

// C(m, n) = sum_k A(m, k) B(n, k) on layer-dtype operands (fp32 C), dispatched on the dtype.
struct Sg {
    const void* A;
    int64_t sam, sak;
    const void* B;
    int64_t sbn, sbk, b_group;
    float* C;
    int64_t scm, c_group;
    int64_t M, N, K;
    const int32_t* offsets;
    int G, mode;
};
void run_sg(const moe_shape* s, const Sg& g, int64_t max_rows, hipStream_t st) {
    if (s->dtype == MOE_BF16) {
        moe::SgArgs a{static_cast<const uint16_t*>(g.A), static_cast<const uint16_t*>(g.B), g.C, g.sam, g.sak, g.sbn,
                      g.sbk, g.scm, g.b_group, g.c_group, g.M, g.N, g.K, g.offsets, 0, g.G, g.mode};
        moe::launch_sg_gemm_bf16(a, max_rows, st);
    } else {
        moe::SgArgsF a{static_cast<const float*>(g.A), static_cast<const float*>(g.B), g.C, g.sam, g.sak, g.sbn,
                       g.sbk, g.scm, g.b_group, g.c_group, g.M, g.N, g.K, g.offsets, 0, g.G, g.mode};
        moe::launch_sg_gemm_f32(a, max_rows, st);
    }
}

struct BwdIn {
    const void *x, *w_in, *b_in, *w_out, *b_out, *ws_in, *ws_out, *x_perm, *y_perm, *dy;
    const float *w_router, *logits, *topk_w;
    const int32_t *topk_idx, *counts, *offsets, *inv_pos;
    float aux_coef;
};
struct BwdOut {
    void* dx;
    float *dw_router, *dw_in, *db_in, *dw_out, *db_out, *dws_in, *dws_out, *dlogits;
};

void do_backward(const moe_shape* s, const BwdIn& in, const BwdOut& out, void* ws, hipStream_t st) {
    const BwdWs w = bwd_ws(s);
    const int64_t T = s->T, A = s->T * s->k, d = s->d_model, F = s->d_ff, E = s->E;
    const int64_t n_in = s->act == MOE_SWIGLU ? 2 * F : F, Fs = s->d_ff_shared;
    const int dt = s->dtype;
    float* dg = at<float>(ws, w.dg);
    void* dYp = at<void>(ws, w.dYp);
    void* pre = at<void>(ws, w.pre);
    void* h = at<void>(ws, w.h);
    float* dh = at<float>(ws, w.dh);
    void* dAU = at<void>(ws, w.dAU);
    float* dXp = at<float>(ws, w.dXp);
    float* dx32 = at<float>(ws, w.dx32);
    float* dl = out.dlogits ? out.dlogits : at<float>(ws, w.dl);
    float* partials = partials_of(ws, w.partials, s);
    // combine: gate gradients and the gate-scaled output gradient per permuted row
    moe::launch_bwd_combine(dt, in.dy, in.y_perm, in.inv_pos, in.topk_w, T, (int)d, s->k, dg, dYp, st);
    // recompute the pre-activations and h of every expert
    const moe::GemmPlan p = moe::plan_gemm(dt, A / E, (int)n_in, (int)d);
    moe::launch_grouped_gemm(dt, moe::EPI_BIAS, p.bm, in.x_perm, in.w_in, in.b_in, pre, in.offsets, 0, (int)E, A, 0,
                             (int)n_in, (int)d, partials, st);
    moe::launch_bwd_act_fwd(dt, pre, A, (int)F, s->act, h, st);
    if (bwd_dgrad_transposed(s)) {
        // dh = dY W_out and dX = dAU W_in on the persistent GEMM (fp32 epilogue), whose operands are
        // both contiguous along K: W_out [E][d][F] -> [E][F][d], W_in [E][n_in][d] -> [E][d][n_in]
        void* w_outT = at<void>(ws, w.w_outT);
        void* w_inT = at<void>(ws, w.w_inT);
        moe::launch_transpose_bf16(in.w_out, E, d, F, w_outT, st);
        moe::launch_transpose_bf16(in.w_in, E, n_in, d, w_inT, st);
        moe::launch_grouped_gemm(dt, moe::EPI_F32, 256, dYp, w_outT, nullptr, dh, in.offsets, 0, (int)E, A, 0, (int)F,
                                 (int)d, partials, st);
        moe::launch_bwd_act_bwd(dt, dh, pre, A, (int)F, s->act, dAU, st);
        moe::launch_grouped_gemm(dt, moe::EPI_F32, 256, dAU, w_inT, nullptr, dXp, in.offsets, 0, (int)E, A, 0, (int)d,
                                 (int)n_in, partials, st);
    } else {
        // dh = dY W_out, then the activation backward
        run_sg(s, Sg{dYp, d, 1, in.w_out, 1, F, d * F, dh, F, 0, 0, F, d, in.offsets, (int)E, moe::SG_ROWS}, A, st);
        moe::launch_bwd_act_bwd(dt, dh, pre, A, (int)F, s->act, dAU, st);
        // dX = dAU W_in
        run_sg(s, Sg{dAU, n_in, 1, in.w_in, 1, d, n_in * d, dXp, d, 0, 0, d, n_in, in.offsets, (int)E, moe::SG_ROWS},
               A, st);
    }
    // weight gradients: K runs over each expert's rows
    if (bwd_wgrad_kgrouped(s)) {
        // transposed copies, each expert's rows a zero-padded column range; then one K-grouped product
        // per weight: dW_out[e] = dY_e^T h_e, dW_in[e] = dAU_e^T X_e
        const int64_t ld = bwd_wgrad_ld(s);
        const int nblk = (int)(ld / 64);
        int32_t* poff = at<int32_t>(ws, w.poff);
        int32_t* pblk = at<int32_t>(ws, w.pblk);
        void* wT1 = at<void>(ws, w.wT1);
        void* wT2 = at<void>(ws, w.wT2);
        moe::launch_wgrad_pad_offsets(in.offsets, (int)E, nblk, poff, pblk, st);
        moe::launch_transpose_pad(dYp, d, in.offsets, poff, pblk, nblk, ld, wT1, st);
        moe::launch_transpose_pad(h, F, in.offsets, poff, pblk, nblk, ld, wT2, st);
        moe::launch_wgrad_kgrouped(wT1, wT2, out.dw_out, poff, (int)E, (int)d, (int)F, ld, st);
        moe::launch_transpose_pad(dAU, n_in, in.offsets, poff, pblk, nblk, ld, wT1, st);
        moe::launch_transpose_pad(in.x_perm, d, in.offsets, poff, pblk, nblk, ld, wT2, st);
        moe::launch_wgrad_kgrouped(wT1, wT2, out.dw_in, poff, (int)E, (int)n_in, (int)d, ld, st);
    } else {
        run_sg(s, Sg{dYp, 1, d, h, 1, F, 0, out.dw_out, F, d * F, d, F, 0, in.offsets, (int)E, moe::SG_KSPLIT}, A,
               st);
        run_sg(s, Sg{dAU, 1, n_in, in.x_perm, 1, d, 0, out.dw_in, d, n_in * d, n_in, d, 0, in.offsets, (int)E,
                     moe::SG_KSPLIT},
               A, st);
    }
    if (out.db_out) moe::launch_bwd_colsum(dt, dYp, in.offsets, 0, (int)E, (int)d, out.db_out, st);
    if (out.db_in) moe::launch_bwd_colsum(dt, dAU, in.offsets, 0, (int)E, (int)F, out.db_in, st);
    // shared expert (gate 1, input x, output gradient dy)
    float* dXs = nullptr;
    if (Fs > 0) {
        void* pre_s = at<void>(ws, w.pre_s);
        void* hs = at<void>(ws, w.hs);
        float* dhs = at<float>(ws, w.dhs);
        void* dAUs = at<void>(ws, w.dAUs);
        dXs = at<float>(ws, w.dXs);
        const moe::GemmPlan ps = moe::plan_gemm(dt, T, (int)(2 * Fs), (int)d);
        moe::launch_grouped_gemm(dt, moe::EPI_BIAS, ps.bm, in.x, in.ws_in, nullptr, pre_s, nullptr, 0, 1, T, T,
                                 (int)(2 * Fs), (int)d, partials, st);
        moe::launch_bwd_act_fwd(dt, pre_s, T, (int)Fs, MOE_SWIGLU, hs, st);
        run_sg(s, Sg{in.dy, d, 1, in.ws_out, 1, Fs, 0, dhs, Fs, 0, T, Fs, d, nullptr, 1, moe::SG_DENSE}, T, st);
        moe::launch_bwd_act_bwd(dt, dhs, pre_s, T, (int)Fs, MOE_SWIGLU, dAUs, st);
        run_sg(s, Sg{dAUs, 2 * Fs, 1, in.ws_in, 1, d, 0, dXs, d, 0, T, d, 2 * Fs, nullptr, 1, moe::SG_DENSE}, T, st);
        run_sg(s, Sg{in.dy, 1, d, hs, 1, Fs, 0, out.dws_out, Fs, 0, d, Fs, T, nullptr, 1, moe::SG_DENSE}, T, st);
        run_sg(s, Sg{dAUs, 1, 2 * Fs, in.x, 1, d, 0, out.dws_in, d, 0, 2 * Fs, d, T, nullptr, 1, moe::SG_DENSE}, T,
               st);
    }
    moe::launch_bwd_unpermute(dXp, in.inv_pos, dXs, T, (int)d, s->k, dx32, st);
    // router: logit gradient through the gates (+ balancing term), then dW_r and dx
    moe::launch_bwd_gate(in.logits, in.topk_idx, dg, in.counts, in.aux_coef, T, (int)E, s->k, s->score, s->renorm, dl,
                         st);
    moe::launch_bwd_router(dt, dl, in.x, in.w_router, dx32, T, (int)E, (int)d, at<float>(ws, w.rpart), out.dw_router,
                           out.dx, st);
}

#define MOE_REQUIRE(cond)                       \
    do {                                        \
        if (!(cond)) return MOE_ERR_INVALID_ARG; \
    } while (0)

inline bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
inline bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

}  // namespace

extern "C" {

int moe_workspace_bytes(const moe_shape* shape, int stage, size_t* bytes) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
    switch (stage) {
        case MOE_STAGE_ROUTE: *bytes = route_ws(shape).bytes; break;
        case MOE_STAGE_PERMUTE: *bytes = perm_ws(shape).bytes; break;
        case MOE_STAGE_FFN: *bytes = ffn_ws(shape).bytes; break;
        case MOE_STAGE_SHARED: *bytes = shared_ws(shape).bytes; break;
        case MOE_STAGE_FORWARD: *bytes = fwd_ws(shape).bytes; break;
        case MOE_STAGE_EXPERT: *bytes = expert_ws(shape).bytes; break;
        case MOE_STAGE_ROUTE_NOISY: *bytes = route_noisy_ws(shape).bytes; break;
        case MOE_STAGE_BACKWARD: *bytes = bwd_ws(shape).bytes; break;
        default: return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

int moe_route(const moe_shape* shape, const void* x, const float* w_router, const float* sel_bias, float* logits,
              int32_t* topk_idx, float* topk_w, int32_t* counts, float* stats, void* ws, size_t ws_bytes,
              moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(ok_ptr(x) && ok_ptr(w_router) && ok_ptr(topk_idx) && ok_ptr(topk_w) && ok_ptr(counts));
    MOE_REQUIRE(ok_opt(sel_bias) && ok_opt(logits) && ok_opt(stats) && ok_opt(ws));
    if (ws_bytes < route_ws(shape).bytes || (ws == nullptr && route_ws(shape).bytes > 0)) return MOE_ERR_WORKSPACE;
    if (shape->T == 0) return MOE_OK;
    (void)hipGetLastError();
    do_route(shape, x, w_router, sel_bias, logits, topk_idx, topk_w, counts, stats, ws,
             static_cast<hipStream_t>(stream));
    return launched();
}

int moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* offsets,
                int32_t* sorted_token, int32_t* inv_pos, void* x_perm, void* ws, size_t ws_bytes,
                moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(ok_ptr(topk_idx) && ok_ptr(x) && ok_ptr(offsets) && ok_ptr(sorted_token) && ok_ptr(inv_pos) &&
                ok_opt(x_perm) && ok_opt(ws));
    if (ws_bytes < perm_ws(shape).bytes || (ws == nullptr && perm_ws(shape).bytes > 0)) return MOE_ERR_WORKSPACE;
    if (shape->T == 0) return MOE_OK;
    (void)hipGetLastError();
    do_permute(shape, topk_idx, x, offsets, sorted_token, inv_pos, x_perm, ws, static_cast<hipStream_t>(stream));
    return launched();
}

int moe_grouped_ffn(const moe_shape* shape, int32_t e_begin, int32_t e_end, const void* x_perm,
                    const int32_t* offsets, const void* w_in, const void* b_in, const void* w_out, const void* b_out,
                    void* y_perm, void* ws, size_t ws_bytes, moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(e_begin >= 0 && e_begin <= e_end && e_end <= shape->E);
    MOE_REQUIRE(ok_ptr(x_perm) && ok_ptr(offsets) && ok_ptr(w_in) && ok_ptr(w_out) && ok_ptr(y_perm) && ok_opt(ws));
    MOE_REQUIRE(ok_opt(b_in) && ok_opt(b_out));
    if (shape->act == MOE_SWIGLU && (b_in != nullptr || b_out != nullptr)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < ffn_ws(shape).bytes || ws == nullptr) return MOE_ERR_WORKSPACE;
    if (shape->T == 0 || e_begin == e_end) return MOE_OK;
    (void)hipGetLastError();
    do_ffn(shape, e_begin, e_end, x_perm, offsets, w_in, b_in, w_out, b_out, y_perm, ws,
           static_cast<hipStream_t>(stream));
    return launched();
}

int moe_expert_up(const moe_shape* shape, int32_t e_begin, int32_t e_end, const void* x_perm, const int32_t* offsets,
                  const void* w_in, const void* b_in, void* h, void* ws, size_t ws_bytes, moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(e_begin >= 0 && e_begin <= e_end && e_end <= shape->E);
    MOE_REQUIRE(ok_ptr(x_perm) && ok_ptr(offsets) && ok_ptr(w_in) && ok_opt(b_in) && ok_ptr(h) && ok_opt(ws));
    if (shape->act == MOE_SWIGLU && b_in != nullptr) return MOE_ERR_INVALID_ARG;
    const ExpertWs w = expert_ws(shape);
    if (ws_bytes < w.bytes || (ws == nullptr && w.bytes > 0)) return MOE_ERR_WORKSPACE;
    if (shape->T == 0 || e_begin == e_end) return MOE_OK;
    (void)hipGetLastError();
    do_up(shape, e_begin, e_end, x_perm, offsets, w_in, b_in, h, partials_of(ws, w.partials, shape),
          static_cast<hipStream_t>(stream));
    return launched();
}

int moe_expert_down(const moe_shape* shape, int32_t e_begin, int32_t e_end, const void* h, const int32_t* offsets,
                    const void* w_out, const void* b_out, void* y_perm, void* ws, size_t ws_bytes,
                    moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(e_begin >= 0 && e_begin <= e_end && e_end <= shape->E);
    MOE_REQUIRE(ok_ptr(h) && ok_ptr(offsets) && ok_ptr(w_out) && ok_opt(b_out) && ok_ptr(y_perm) && ok_opt(ws));
    if (shape->act == MOE_SWIGLU && b_out != nullptr) return MOE_ERR_INVALID_ARG;
    const ExpertWs w = expert_ws(shape);
    if (ws_bytes < w.bytes || (ws == nullptr && w.bytes > 0)) return MOE_ERR_WORKSPACE;
    if (shape->T == 0 || e_begin == e_end) return MOE_OK;
    (void)hipGetLastError();
    do_down(shape, e_begin, e_end, h, offsets, w_out, b_out, y_perm, partials_of(ws, w.partials, shape),
            static_cast<hipStream_t>(stream));
    return launched();
}

int moe_shared_ffn(const moe_shape* shape, const void* x, const void* ws_in, const void* ws_out, void* y_shared,
                   void* ws, size_t ws_bytes, moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->d_ff_shared == 0) return MOE_ERR_INVALID_ARG;
    MOE_REQUIRE(ok_ptr(x) && ok_ptr(ws_in) && ok_ptr(ws_out) && ok_ptr(y_shared) && ok_opt(ws));
    if (ws_bytes < shared_ws(shape).bytes || (ws == nullptr && shared_ws(shape).bytes > 0)) return MOE_ERR_WORKSPACE;
    if (shape->T == 0) return MOE_OK;
    (void)hipGetLastError();
    do_shared(shape, x, ws_in, ws_out, y_shared, ws, static_cast<hipStream_t>(stream));
    return launched();
}

int moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                const void* y_shared, void* y, moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(ok_ptr(y_perm) && ok_ptr(inv_pos) && ok_ptr(topk_w) && ok_opt(y_shared) && ok_ptr(y));
    if (shape->T == 0) return MOE_OK;
    (void)hipGetLastError();
    moe::launch_combine(shape->dtype, y_perm, inv_pos, topk_w, y_shared, y, shape->T, shape->d_model, shape->k,
                        static_cast<hipStream_t>(stream));
    return launched();
}

int moe_route_noisy(const moe_shape* shape, const void* x, const float* w_router, const float* w_noise,
                    const float* noise, const float* sel_bias, float* logits, int32_t* topk_idx, float* topk_w,
                    int32_t* counts, float* stats, void* ws, size_t ws_bytes, moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(ok_ptr(x) && ok_ptr(w_router) && ok_ptr(w_noise) && ok_ptr(noise) && ok_ptr(topk_idx) &&
                ok_ptr(topk_w) && ok_ptr(counts));
    MOE_REQUIRE(ok_opt(sel_bias) && ok_opt(logits) && ok_opt(stats) && ok_opt(ws));
    const size_t need = route_noisy_ws(shape).bytes;
    if (ws_bytes < need || (ws == nullptr && need > 0)) return MOE_ERR_WORKSPACE;
    if (shape->T == 0) return MOE_OK;
    (void)hipGetLastError();
    do_route_noisy(shape, x, w_router, w_noise, noise, sel_bias, logits, topk_idx, topk_w, counts, stats, ws,
                   static_cast<hipStream_t>(stream));
    return launched();
}

int moe_update_bias(const moe_shape* shape, const int32_t* counts, float gamma, float* sel_bias,
                    moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(ok_ptr(counts) && ok_ptr(sel_bias) && std::isfinite(gamma));
    (void)hipGetLastError();
    moe::launch_route_bias_update(counts, shape->T, shape->E, shape->k, gamma, sel_bias,
                                  static_cast<hipStream_t>(stream));
    return launched();
}

int moe_forward(const moe_shape* shape, const void* x, const float* w_router, const float* sel_bias,
                const void* w_in, const void* b_in, const void* w_out, const void* b_out, const void* ws_in,
                const void* ws_out, void* y, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                float* stats_out, void* ws, size_t ws_bytes, moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    MOE_REQUIRE(ok_ptr(x) && ok_ptr(w_router) && ok_opt(sel_bias) && ok_ptr(w_in) && ok_ptr(w_out) && ok_ptr(y));
    MOE_REQUIRE(ok_opt(b_in) && ok_opt(b_out) && ok_opt(topk_idx_out) && ok_opt(topk_w_out) &&
                ok_opt(counts_out) && ok_opt(stats_out) && ok_opt(ws));
    if (shape->act == MOE_SWIGLU && (b_in != nullptr || b_out != nullptr)) return MOE_ERR_INVALID_ARG;
    if (shape->d_ff_shared > 0) MOE_REQUIRE(ok_ptr(ws_in) && ok_ptr(ws_out));
    else MOE_REQUIRE(ws_in == nullptr && ws_out == nullptr);
    const FwdWs w = fwd_ws(shape);
    if (ws_bytes < w.bytes || ws == nullptr) return MOE_ERR_WORKSPACE;
    if (shape->T == 0) return MOE_OK;
    (void)hipGetLastError();
    const hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, w.topk_idx);
    float* gw = topk_w_out ? topk_w_out : at<float>(ws, w.topk_w);
    int32_t* cnt = counts_out ? counts_out : at<int32_t>(ws, w.counts);
    void* scratch = at<void>(ws, w.scratch);
    int32_t* offsets = at<int32_t>(ws, w.offsets);
    int32_t* inv_pos = at<int32_t>(ws, w.inv_pos);
    do_route(shape, x, w_router, sel_bias, nullptr, idx, gw, cnt, stats_out, scratch, st);
    int32_t* sorted_token = at<int32_t>(ws, w.sorted_token);
    if (fwd_gathers(shape)) {  // positions only; the up projection gathers the token rows itself
        do_permute(shape, idx, x, offsets, sorted_token, inv_pos, nullptr, scratch, st);
        do_ffn(shape, 0, shape->E, x, offsets, w_in, b_in, w_out, b_out, at<void>(ws, w.y_perm), scratch, st,
               sorted_token);
    } else {
        do_permute(shape, idx, x, offsets, sorted_token, inv_pos, at<void>(ws, w.x_perm), scratch, st);
        do_ffn(shape, 0, shape->E, at<void>(ws, w.x_perm), offsets, w_in, b_in, w_out, b_out, at<void>(ws, w.y_perm),
               scratch, st);
    }
    void* ys = nullptr;
    if (shape->d_ff_shared > 0) {
        ys = at<void>(ws, w.ys);
        do_shared(shape, x, ws_in, ws_out, ys, scratch, st);
    }
    moe::launch_combine(shape->dtype, at<void>(ws, w.y_perm), inv_pos, gw, ys, y, shape->T, shape->d_model, shape->k,
                        st);
    return launched();
}

int moe_backward(const moe_shape* shape, const void* x, const float* w_router, const void* w_in, const void* b_in,
                 const void* w_out, const void* b_out, const void* ws_in, const void* ws_out, const float* logits,
                 const int32_t* topk_idx, const float* topk_w, const int32_t* counts, const int32_t* offsets,
                 const int32_t* inv_pos, const void* x_perm, const void* y_perm, const void* dy, float aux_coef,
                 void* dx, float* dw_router, float* dw_in, float* db_in, float* dw_out, float* db_out,
                 float* dws_in, float* dws_out, float* dlogits, void* ws, size_t ws_bytes, moe_stream_t stream) {
    const int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    // the backward's bf16 products and transposes tile d_model and the hidden sizes by 64
    if (shape->dtype == MOE_BF16 && (shape->d_model % 64 || shape->d_ff % 64 || shape->d_ff_shared % 64))
        return MOE_ERR_UNSUPPORTED;
    MOE_REQUIRE(ok_ptr(x) && ok_ptr(w_router) && ok_ptr(w_in) && ok_ptr(w_out) && ok_ptr(logits) && ok_ptr(topk_idx) &&
                ok_ptr(topk_w) && ok_ptr(offsets) && ok_ptr(inv_pos) && ok_ptr(x_perm) && ok_ptr(y_perm) &&
                ok_ptr(dy));
    MOE_REQUIRE(ok_ptr(dx) && ok_ptr(dw_router) && ok_ptr(dw_in) && ok_ptr(dw_out) && ok_opt(dlogits) && ok_opt(ws));
    MOE_REQUIRE(ok_opt(b_in) && ok_opt(b_out) && ok_opt(db_in) && ok_opt(db_out) && ok_opt(counts));
    MOE_REQUIRE(std::isfinite(aux_coef));
    if (aux_coef != 0.f) MOE_REQUIRE(counts != nullptr);
    if (shape->act == MOE_SWIGLU && (b_in != nullptr || b_out != nullptr)) return MOE_ERR_INVALID_ARG;
    // a bias gradient exactly when the bias exists
    MOE_REQUIRE((b_in == nullptr) == (db_in == nullptr) && (b_out == nullptr) == (db_out == nullptr));
    if (shape->d_ff_shared > 0) MOE_REQUIRE(ok_ptr(ws_in) && ok_ptr(ws_out) && ok_ptr(dws_in) && ok_ptr(dws_out));
    else MOE_REQUIRE(ws_in == nullptr && ws_out == nullptr && dws_in == nullptr && dws_out == nullptr);
    const BwdWs w = bwd_ws(shape);
    if (ws_bytes < w.bytes || ws == nullptr) return MOE_ERR_WORKSPACE;
    if (shape->T == 0) return MOE_OK;
    (void)hipGetLastError();
    const BwdIn in{x, w_in, b_in, w_out, b_out, ws_in, ws_out, x_perm, y_perm, dy, w_router, logits, topk_w,
                   topk_idx, counts, offsets, inv_pos, aux_coef};
    const BwdOut out{dx, dw_router, dw_in, db_in, dw_out, db_out, dws_in, dws_out, dlogits};
    do_backward(shape, in, out, ws, static_cast<hipStream_t>(stream));
    return launched();
}

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

}  // extern "C"

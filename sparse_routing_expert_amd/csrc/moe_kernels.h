// Host-side launchers of the libmoe kernels (internal; the public ABI is include/moe.h).
// Every launcher only enqueues work on `stream`; argument checks happen in moe_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- route ------------------------------------------------------------------------------
constexpr int kRouteTokensPerBlock = 16;  // tokens per select block (4 waves x 4 tokens)

// bf16 layers: split the fp32 router into hi/mid/lo bf16 rows [3][Epad][d] (rows >= E zero);
// every layer: zero the statistics ticket.
void launch_route_prep(const float* w_router, int E, int Epad, int d, uint16_t* wsplit, int32_t* ticket,
                       hipStream_t s);
void launch_route_logits(int dtype, const void* x, const float* w_router, const uint16_t* wsplit, int Epad,
                         float* logits, int64_t T, int d, int E, hipStream_t s);
// s_logits / noise (both or neither): noisy top-k, logits replaced by logits + noise * softplus(s_logits),
// written to h_out when given
void launch_route_select(const float* logits, const float* sel_bias, int64_t T, int E, int k, int score,
                         int renorm, int32_t* topk_idx, float* topk_w, int32_t* blk_counts, float* blk_P,
                         float* blk_H, const float* s_logits, const float* noise, float* h_out, hipStream_t s);
// counts[E] always; stats (f, P, aux, entropy) when stats != NULL
void launch_route_finalize(const int32_t* blk_counts, const float* blk_P, const float* blk_H, int nblk, int64_t T,
                           int E, int32_t* counts, double* fp_scratch, int32_t* ticket, float* stats,
                           hipStream_t s);

// sel_bias[e] -= gamma * sign(counts[e] * E - T * k)
void launch_route_bias_update(const int32_t* counts, int64_t T, int E, int k, float gamma, float* sel_bias,
                              hipStream_t s);

// ---- permute ----------------------------------------------------------------------------
constexpr int kPermTile = 1024;  // assignments per histogram / rank tile

void launch_perm_count(const int32_t* topk_idx, int64_t A, int E, int32_t* tile_counts, hipStream_t s);
// capacity: rows each expert keeps (0 = all); dropped assignments get inv_pos = -1
void launch_perm_scan(const int32_t* tile_counts, int ntiles, int64_t A, int E, int capacity, int32_t* tile_base,
                      int32_t* offsets, hipStream_t s);
void launch_perm_rank(const int32_t* topk_idx, const int32_t* tile_base, const int32_t* offsets, int64_t A, int E,
                      int k, int capacity, int32_t* inv_pos, int32_t* sorted_token, hipStream_t s);
void launch_perm_scatter(const void* x, const int32_t* inv_pos, int64_t T, int d, int k, int elem_bytes,
                         void* x_perm, hipStream_t s);

// ---- grouped FFN ------------------------------------------------------------------------
enum Epilogue { EPI_SWIGLU = 0, EPI_GELU_BIAS = 1, EPI_BIAS = 2 };

struct GemmPlan {
    int bm;  // rows per tile
};
GemmPlan plan_gemm(int dtype, int64_t rows_per_group_hint, int n_out, int K);

// C[rows, n_out] = epi(A[rows, K] * B_e^T) over groups e_begin.. (offsets != NULL; the kernel builds
// its tile schedule from the device-side offsets) or one dense group of `dense_rows` rows
// (offsets == NULL). B is [E][n_b_rows][K] (n_b_rows = 2*n_out for SwiGLU). One kernel launch.
// partials: fp32 scratch of gemm_partials_bytes(dtype) bytes (or NULL) in which the bf16 kernel
// splits the last, incomplete round of tiles along K; summed in a fixed order by a second launch.
void launch_grouped_gemm(int dtype, int epi, int bm, const void* A, const void* B, const void* bias,
                         void* C, const int32_t* offsets, int e_begin, int n_groups, int64_t max_rows,
                         int64_t dense_rows, int n_out, int K, float* partials, hipStream_t s);
size_t gemm_partials_bytes(int dtype);

// ---- combine ----------------------------------------------------------------------------
void launch_combine(int dtype, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                    const void* y_shared, void* y, int64_t T, int d, int k, hipStream_t s);

}  // namespace moe

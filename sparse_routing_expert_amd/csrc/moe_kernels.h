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
// Logits (and s_logits) of token t, expert e at [t * lg_ld + e], or, with lg_split > 0, the sum of the
// split-router products at columns e, lg_split + e, 2 * lg_split + e (written to logits_out when given).
// s_logits / noise (both or neither): noisy top-k, logits replaced by logits + noise * softplus(s_logits),
// written to h_out when given
void launch_route_select(const float* logits, int lg_ld, int lg_split, float* logits_out, const float* sel_bias,
                         int64_t T, int E, int k, int score, int renorm, int32_t* topk_idx, float* topk_w,
                         int32_t* blk_counts, float* blk_P, float* blk_H, const float* s_logits, const float* noise,
                         float* h_out, hipStream_t s);
// Routers with at least this many (16-padded) experts take the logits as one dense MFMA product
// x [T, d] . [hi; mid; lo]^T [3 Epad, d] through the grouped GEMM (fp32 output), split along K over
// every CU; the select kernel sums the three products.
constexpr int kRouteGemmMinEpad = 64;
// Small routers (route_small_ok): logits (written to `logits` when given), selection and per-block
// partials in one launch over blocks of route_small_tokens_per_block(T, E, noisy) tokens; zeroes *ticket.
bool route_small_ok(int dtype, int E, int k, int d);
int route_small_tokens_per_block(int64_t T, int E, bool noisy);
void launch_route_small(const void* x, const float* w_router, const float* w_noise, const float* noise,
                        const float* sel_bias, int64_t T, int d, int E, int k, int score, int renorm, float* logits,
                        int32_t* topk_idx, float* topk_w, int32_t* blk_counts, float* blk_P, float* blk_H,
                        int32_t* ticket, hipStream_t s);
// counts[E] always; stats (f, P, aux, entropy) when stats != NULL
void launch_route_finalize(const int32_t* blk_counts, const float* blk_P, const float* blk_H, int nblk, int64_t T,
                           int E, int32_t* counts, double* fp_scratch, int32_t* ticket, float* stats,
                           hipStream_t s);

// sel_bias[e] -= gamma * sign(counts[e] * E - T * k)
void launch_route_bias_update(const int32_t* counts, int64_t T, int E, int k, float gamma, float* sel_bias,
                              hipStream_t s);

// ---- permute ----------------------------------------------------------------------------
constexpr int kPermTile = 1024;  // assignments per histogram / rank tile
// the scatter forms the offsets and tile bases itself for at most this many experts and tiles
constexpr int kPermFoldExperts = 64;
constexpr int kPermFoldTiles = 64;
// single-block index stage: per-chunk (64 assignments) expert counts held in LDS
constexpr int kPermSmallCounts = 16384;
// A <= 16 waves x 4 chunks x 64 = 4096. Measured beyond that, the one block is slower than the tiled
// kernels (A = 16384: 62.9 us for the permute, against 56.4 us for the four-launch tiled path of the
// time and 47 us for the two-launch one; A = 8192: even with the four-launch path)
constexpr int kPermSmallChunksPerWave = 4;
// with at most kPermFoldExperts experts the single block is used up to this many assignments
// (measured cold: A = 2048, 13.9 against 14.3 us for the tiled path; A = 4096, 19.8 against 17.8 us)
constexpr int kPermSmallFoldMax = 2048;
// Tiled index path: perm_local (tile counts, in-tile ranks into inv_pos), then perm_scan unless
// perm_fold_ok (tile_base == nullptr: the scatter forms offsets and bases itself), then the placing
// scatter (inv_pos, sorted_token, x_perm; offsets when folded).
void launch_perm_local(const int32_t* topk_idx, int64_t A, int E, int32_t* tile_counts, int32_t* local_rank,
                       hipStream_t s);
bool perm_fold_ok(int64_t A, int E, int k);
void launch_perm_place_scatter(const void* x, const int32_t* topk_idx, const int32_t* tile_counts,
                               const int32_t* tile_base, int32_t* offsets, int E, int capacity, int64_t T, int d,
                               int k, int elem_bytes, int32_t* inv_pos, int32_t* sorted_token, void* x_perm,
                               hipStream_t s);
bool perm_index_small_ok(int64_t A, int E);
void launch_perm_index_small(const int32_t* topk_idx, int64_t A, int E, int k, int capacity, int32_t* offsets,
                             int32_t* inv_pos, int32_t* sorted_token, hipStream_t s);

// capacity: rows each expert keeps (0 = all); dropped assignments get inv_pos = -1
void launch_perm_scan(const int32_t* tile_counts, int ntiles, int64_t A, int E, int capacity, int32_t* tile_base,
                      int32_t* offsets, hipStream_t s);
void launch_perm_scatter(const void* x, const int32_t* inv_pos, int64_t T, int d, int k, int elem_bytes,
                         void* x_perm, hipStream_t s);

// ---- grouped FFN ------------------------------------------------------------------------
// EPI_F32 (dense bf16 products only): C is float, the fp32 accumulators stored as they are
enum Epilogue { EPI_SWIGLU = 0, EPI_GELU_BIAS = 1, EPI_BIAS = 2, EPI_F32 = 3 };

struct GemmPlan {
    int bm;  // rows per tile
};
#ifndef MOE_GEMM_SMALL_ROWS_MAX
#define MOE_GEMM_SMALL_ROWS_MAX 32
#endif
// bf16 grouped products whose groups average at most this many rows take 64-row tiles
constexpr int64_t kGemmSmallRowsMax = MOE_GEMM_SMALL_ROWS_MAX;
GemmPlan plan_gemm(int dtype, int64_t rows_per_group_hint, int n_out, int K);

// C[rows, n_out] = epi(A[rows, K] * B_e^T) over groups e_begin.. (offsets != NULL; the kernel builds
// its tile schedule from the device-side offsets) or one dense group of `dense_rows` rows
// (offsets == NULL). B is [E][n_b_rows][K] (n_b_rows = 2*n_out for SwiGLU). One kernel launch.
// partials: fp32 scratch of gemm_partials_bytes(dtype) bytes (or NULL) in which the bf16 kernel
// splits the last, incomplete round of tiles along K; summed in a fixed order by a second launch.
// gather (bf16 only, with EPI_SWIGLU or EPI_GELU_BIAS; NULL = A's rows in order): A is then a
// [a_rows, K] token matrix and row p of the product's input is A[gather[p]] (a_rows * K * 2 < 2^31
// bytes), read straight into the GEMM's LDS ring, so no permuted copy of A is written. The gather
// buffer must hold 256 readable entries past the last row.
void launch_grouped_gemm(int dtype, int epi, int bm, const void* A, const void* B, const void* bias,
                         void* C, const int32_t* offsets, int e_begin, int n_groups, int64_t max_rows,
                         int64_t dense_rows, int n_out, int K, float* partials, hipStream_t s,
                         const int32_t* gather = nullptr, int64_t a_rows = 0);
size_t gemm_partials_bytes(int dtype);

// ---- combine ----------------------------------------------------------------------------
void launch_combine(int dtype, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                    const void* y_shared, void* y, int64_t T, int d, int k, hipStream_t s);

// ---- backward ---------------------------------------------------------------------------
// bf16 [G][R][C] -> [G][C][R] (R, C multiples of 64)
void launch_transpose_bf16(const void* src, int64_t G, int64_t R, int64_t C, void* dst, hipStream_t s);
// weight gradients on the wide GEMM: per-expert K offsets of the transposed copies, padded to 64
// (poff [E + 1], blk [nblk] = owning expert of each 64-column block or -1), the padded transposes
// ([A][C] -> [C][ld], C a multiple of 64), and the K-grouped product dW[e] = A_T[e] B_T[e]^T
// (fp32 [E * m_per_e][n_out], m_per_e a multiple of 256)
void launch_wgrad_pad_offsets(const int32_t* offsets, int E, int nblk, int32_t* poff, int32_t* blk, hipStream_t s);
void launch_transpose_pad(const void* src, int64_t C, const int32_t* offsets, const int32_t* poff,
                          const int32_t* blk, int nblk, int64_t ld, void* dst, hipStream_t s);
void launch_wgrad_kgrouped(const void* AT, const void* BT, float* C, const int32_t* poff, int E, int m_per_e,
                           int n_out, int64_t ld, hipStream_t s);
// Strided grouped GEMM C(m, n) = sum_k A(m, k) B(n, k); A(m, k) at A[m*sam + k*sak], B(n, k) at
// B[n*sbn + k*sbk], C(m, n) at C[m*scm + n] (fp32). Each operand is contiguous along k (s?k == 1) or
// along its row index (sam == 1 / sbn == 1).
//   SG_ROWS:   group g = expert e_begin + g owns rows offsets[e_begin+g] .. offsets[e_begin+g+1] of
//              A and C; B advances b_group elements per group; N, K fixed (M unused)
//   SG_KSPLIT: group g sums k over offsets[e_begin+g] .. offsets[e_begin+g+1]; C advances c_group
//              elements per group; M, N fixed
//   SG_DENSE:  one group, M x N, k in [0, K)
enum SgMode { SG_ROWS = 0, SG_KSPLIT = 1, SG_DENSE = 2 };
struct SgArgs {
    const uint16_t* A;
    const uint16_t* B;
    float* C;
    int64_t sam, sak, sbn, sbk, scm, b_group, c_group;
    int64_t M, N, K;
    const int32_t* offsets;
    int e_begin, G, mode;
};
struct SgArgsF {
    const float* A;
    const float* B;
    float* C;
    int64_t sam, sak, sbn, sbk, scm, b_group, c_group;
    int64_t M, N, K;
    const int32_t* offsets;
    int e_begin, G, mode;
};
// max_rows: total rows of the grouped buffer (SG_ROWS grid bound). bf16: N and scm multiples of 4 and
// C 16-byte aligned (each lane stores 4 consecutive columns).
void launch_sg_gemm_bf16(const SgArgs& a, int64_t max_rows, hipStream_t s);
void launch_sg_gemm_f32(const SgArgsF& a, int64_t max_rows, hipStream_t s);

// dg[t, j] = <dy[t], y_perm[row]>, dYp[row] = topk_w[t, j] * dy[t] for kept slots (dg = 0 if dropped)
void launch_bwd_combine(int dtype, const void* dy, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                        int64_t T, int d, int k, float* dg, void* dYp, hipStream_t s);
// h = act(pre): SwiGLU pre [rows, 2F] -> silu(a) * u; GELU pre [rows, F] -> gelu(z)
void launch_bwd_act_fwd(int dtype, const void* pre, int64_t n_rows, int F, int act, void* h, hipStream_t s);
// dAU [rows, n_in] from dh [rows, F] fp32 and pre
void launch_bwd_act_bwd(int dtype, const float* dh, const void* pre, int64_t n_rows, int F, int act, void* dAU,
                        hipStream_t s);
// dx32[t] = sum over kept slots of dXp[inv_pos[t*k + j]] (+ extra[t])
void launch_bwd_unpermute(const float* dXp, const int32_t* inv_pos, const float* extra, int64_t T, int d, int k,
                          float* dx32, hipStream_t s);
// out[g][c] = sum of src rows offsets[e_begin+g] .. offsets[e_begin+g+1], column c
void launch_bwd_colsum(int dtype, const void* src, const int32_t* offsets, int e_begin, int G, int ncols, float* out,
                       hipStream_t s);
// router logit gradient [T, E] from the gate gradients (+ the balancing term when aux_coef != 0)
void launch_bwd_gate(const float* logits, const int32_t* topk_idx, const float* dg, const int32_t* counts,
                     float aux_coef, int64_t T, int E, int k, int score, int renorm, float* dl, hipStream_t s);
// dw_r = dl^T x (token chunks of kRouterChunk summed in order through `partials`), dx = dx32 + dl W_r
constexpr int kRouterChunk = 256;
// bf16 grouped GEMM: expert groups averaging at least this many rows use the four-wave wide-K
// persistent kernel (measured: Mixtral-shaped projections, 2048 rows per expert, 2-3 % faster; groups
// of 128 to 1024 rows and a dense 4096-row product slower than on the eight-wave kernel) ...
constexpr int64_t kGemmWideRows = 2048;
// ... and so do groups averaging at least kGemmWideRowsLongK rows over a K of at least kGemmWideMinK
// (measured: Qwen3-shaped gate/up, 1024 rows per expert and K = 2048, 0.913 against 0.952 ms; its
// down projection, K = 768, and the small layer's, K = 1024, are faster on the eight-wave kernel)
constexpr int64_t kGemmWideRowsLongK = 1024;
constexpr int kGemmWideMinK = 2048;
// Groups averaging at most this many rows take the persistent kernel's 128-row tiles (measured:
// DeepSeek-shaped layer, 128 rows per expert, gate/up 3.67 -> 3.55 ms and the step 3.6 % faster; the
// small layer's 512-row groups 7 % slower, so they keep 256-row tiles)
#ifndef MOE_GEMM_R128_ROWS
#define MOE_GEMM_R128_ROWS 256
#endif
constexpr int64_t kGemmR128Rows = MOE_GEMM_R128_ROWS;
// Weight rows per tile of the wide-K kernel: 256, or 384 (the tile schedule then moves from LDS into
// registers, for launches of at most 128 expert groups)
#ifndef MOE_GEMM_WIDE_BN
#define MOE_GEMM_WIDE_BN 384
#endif
constexpr int kGemmWideBN = MOE_GEMM_WIDE_BN;
constexpr int kRouterWgradExperts = 32;  // experts per dW_r block (x read once per 32 experts)
constexpr int kRouterDgradTokens = 16;   // tokens per dx block (W_r read once per 16 tokens)
size_t bwd_router_partials_bytes(int64_t T, int E, int d);
void launch_bwd_router(int dtype, const float* dl, const void* x, const float* w_r, const float* dx32, int64_t T,
                       int E, int d, float* partials, float* dw_r, void* dx, hipStream_t s);

}  // namespace moe

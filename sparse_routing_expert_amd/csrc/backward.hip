// moe_backward kernels: gradients of the MoE-FFN layer (the chain rule of the forward in
// moe_route / moe_permute / moe_grouped_ffn / moe_combine; the fine-tuning setting of "Fine-Tuning
// Mixture of Experts (MoE) Models: Router Optimization Techniques" and "Fine-tuning and serving MoE
// models").
//
// Products with a transposed or token-indexed operand (dh = dY Wd, dX = dAU W_in, dWd = dY^T h,
// dW_in = dAU^T X) all go through one strided grouped GEMM, C(m, n) = sum_k A(m, k) B(n, k) with
// arbitrary element strides, so no operand is ever transposed in memory:
//   rows:   groups are expert segments of a permuted buffer (rows offsets[g] .. offsets[g+1]),
//           B and K per group (dgrad),
//   ksplit: K runs over an expert's rows (k = offsets[g] .. offsets[g+1]), one C per group (wgrad),
//   dense:  one group (the shared expert).
// bf16 operands use v_mfma_f32_32x32x16_bf16 on 128 x 128 tiles with fp32 accumulation and fp32
// output; a 16-byte load runs along whichever of the operand's two indices is contiguous, and the
// LDS tile is always K-contiguous (64-byte rows, XOR-swizzled 16-byte chunks). fp32 operands
// (fp32 layers) take a plain per-element kernel.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe.h"

namespace moe {

namespace {

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float silu_b(float z) { return z * sigm(z); }
__device__ __forceinline__ float silu_grad_b(float z) {
    const float s = sigm(z);
    return s * (1.0f + z * (1.0f - s));
}
__device__ __forceinline__ float gelu_b(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_grad_b(float z) {
    return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) + z * 0.39894228040143268f * expf(-0.5f * z * z);
}

template <bool BF16>
__device__ __forceinline__ float ld_elem(const void* p, int64_t i) {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    return static_cast<const float*>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ void st_elem(void* p, int64_t i, float v) {
    if (BF16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else static_cast<float*>(p)[i] = v;
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Strided grouped GEMM
// ------------------------------------------------------------------------------------------------

// rows mode: the per-block tile schedule (prefix sums of BM-row tiles per group) in LDS.
template <int BM>
__device__ __forceinline__ void sg_schedule(const int32_t* __restrict__ offsets, int e_begin, int G, int* s_ts,
                                            int* s_wave) {
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    int n[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = tid * 4 + i;
        n[i] = 0;
        if (g < G) n[i] = (offsets[e_begin + g + 1] - offsets[e_begin + g] + BM - 1) / BM;
        sum += n[i];
    }
    int inc = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += v;
    }
    if (lane == kWave - 1) s_wave[wave] = inc;
    __syncthreads();
    int base = inc - sum;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = tid * 4 + i;
        if (g < G) s_ts[g] = base;
        base += n[i];
    }
    if (tid == 255) s_ts[G] = base;
    __syncthreads();
}

// LDS element offset of (row R, 16-byte chunk c) inside one stage of 64-byte rows. Rows are permuted
// within each group of four by bits 3-4 of the row and chunks are XOR-swizzled by bits 2-3, so each
// quarter-wave access below covers the 64 banks once: 16 lanes reading 16 consecutive rows at one
// chunk (MFMA fragments), writing 4 consecutive rows x 4 chunks (K-contiguous operand), or writing
// row 8*mg + i of 4 consecutive mg x 4 chunks (transposed operand).
__device__ __forceinline__ int sg_lds(int R, int c) {
    return (((R & ~3) | ((R ^ (R >> 3)) & 3)) << 5) + ((c ^ ((R >> 2) & 3)) << 3);
}

// Row q of the transpose of an 8 x 8 bf16 block held as 8 rows (k = 0..7) of 8 elements (m = 0..7):
// the 8 values of k at m = q, packed as 4 dwords of (k = 2j, 2j + 1).
// (q is a constant after the callers' loops unroll.)
__device__ __forceinline__ u32x4 sg_tr_row(const u32x4* v, int q) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t x = v[2 * j][q >> 1], y = v[2 * j + 1][q >> 1];
        o[j] = (q & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
    }
    return o;
}

// Strided grouped GEMM, bf16 operands, fp32 C. 256 x 256 tiles, four waves of 128 x 128 (4 x 4
// v_mfma_f32_32x32x16_bf16 tiles), BK = 32, two LDS stages and two register staging sets, loads
// issued three stages ahead (the register-staged schedule of the forward GEMM). Waves 0-1 stage
// operand A and waves 2-3 operand B, 8 x 16 bytes per thread and stage. A K-contiguous operand
// (AK / BK_ true) loads 16 bytes along k of one row; a row-contiguous one loads an 8 x 8 block (8
// rows of k, 8 consecutive m each) and writes its transpose. Buffer descriptors bound every load:
// rows past the tile's valid range and k past the group's K read as zero.
template <bool AK, bool BKC>
__global__ __launch_bounds__(256, 1) void sg_gemm_bf16_kernel(SgArgs p) {
    constexpr int BM = 256, BN = 256, BK = 32, TM = 4, TN = 4, NQ = 8;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int STEPS = 16, RNH = 4, RSP = 4;
    static_assert(STEPS >= 2 * NQ && STEPS >= TM + TN && RSP * RNH == STEPS, "schedule slots");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * STAGE];
    int* s_ts = reinterpret_cast<int*>(lds);
    int* s_wave = s_ts + 1025;
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t tiles_n = (p.N + BN - 1) / BN;

    // ---- tile -> (group, m0, n0), the group's M and K range
    int g = 0;
    int64_t m0 = 0, n0 = 0, M = p.M, kb = 0, ke = p.K, row_base = 0;
    if (p.mode == SG_ROWS) {
        sg_schedule<BM>(p.offsets, p.e_begin, p.G, s_ts, s_wave);
        const int64_t lin = blockIdx.x;
        const int64_t total = (int64_t)s_ts[p.G] * tiles_n;
        if (lin >= total) return;  // uniform per block
        const int64_t key = lin / tiles_n;
        int lo = 0, hi = p.G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_ts[mid] <= key) lo = mid;
            else hi = mid - 1;
        }
        g = lo;
        m0 = (key - s_ts[g]) * BM;
        n0 = (lin % tiles_n) * BN;
        row_base = p.offsets[p.e_begin + g];
        M = p.offsets[p.e_begin + g + 1] - row_base;
        __syncthreads();  // the schedule shares LDS with the stages
    } else {
        const int64_t tiles_m = (p.M + BM - 1) / BM;
        const int64_t per_group = tiles_m * tiles_n;
        g = (int)(blockIdx.x / per_group);
        if (g >= p.G) return;
        const int64_t tt = blockIdx.x % per_group;
        m0 = (tt / tiles_n) * BM;
        n0 = (tt % tiles_n) * BN;
        if (p.mode == SG_KSPLIT) {
            kb = p.offsets[p.e_begin + g];
            ke = p.offsets[p.e_begin + g + 1];
        }
    }
    const int64_t Kext = ke - kb;
    const int nk = (int)((Kext + BK - 1) / BK);
    const uint16_t* Ag = p.A + (p.mode == SG_ROWS ? row_base * p.sam : 0);
    const uint16_t* Bg = p.B + (int64_t)(p.mode == SG_ROWS ? g : 0) * p.b_group;
    float* C = p.C + (p.mode == SG_ROWS ? row_base * p.scm : (int64_t)g * p.c_group);

    // ---- this thread's operand: element (row r, k) at X0 + r * s_row + k * s_k, r < rows_valid
    const bool isA = wave < 2;
    const int t = tid & 127;
    const uint16_t* X0 = isA ? Ag + m0 * p.sam + kb * p.sak : Bg + n0 * p.sbn + kb * p.sbk;
    const int64_t s_row = isA ? p.sam : p.sbn, s_k = isA ? p.sak : p.sbk;
    const int64_t rv64 = isA ? M - m0 : p.N - n0;
    const int rows_valid = (int)(rv64 < BM ? rv64 : BM);
    const int lds_row0 = isA ? 0 : BM;
    // K-contiguous: one descriptor for the tile (rows beyond rows_valid read 0), the stage as soffset.
    // Row-contiguous: a descriptor per stage covering k in [k0, min(k0 + BK, Kext)).
    // K-contiguous operands have K a multiple of BK (checked by the host), so only rows need a bound.
    const bool kcont = isA ? AK : BKC;
    const __amdgpu_buffer_rsrc_t rs_tile = __builtin_amdgcn_make_buffer_rsrc(
        (void*)X0, (short)0, kcont && rows_valid > 0 ? (int)(((int64_t)rows_valid - 1) * s_row * 2 + Kext * 2) : 0,
        0x00020000);
    int voff[NQ];
    int wofs[NQ];
    const int mg = t >> 2, kg = t & 3;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (kcont) {
            const int r = q * 32 + (t >> 2), c = t & 3;
            voff[q] = (int)(r * s_row * 2) + c * 16;
            wofs[q] = sg_lds(lds_row0 + r, c);
        } else {
            voff[q] = (int)((mg * 8 + (kg * 8 + q) * s_k) * 2);
            wofs[q] = sg_lds(lds_row0 + mg * 8 + q, kg);
        }
    }
    const int wm = wave & 1, wn = wave >> 1;
    int a_base[TM], a_sw[TM], b_base[TN], b_sw[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * 128 + i * 32 + (lane & 31);
        a_base[i] = sg_lds(r, 0) & ~31;
        a_sw[i] = (r >> 2) & 3;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r = BM + wn * 128 + j * 32 + (lane & 31);
        b_base[j] = sg_lds(r, 0) & ~31;
        b_sw[j] = (r >> 2) & 3;
    }
    const int khalf = lane >> 5;
    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    bf16x8 fa[2][TM], fb[2][TN];
    u32x4 stg[2][NQ];

#define SG_LOAD1(set, q, stage)                                                                           \
    {                                                                                                     \
        if (KC) {                                                                                         \
            stg[set][q] = __builtin_bit_cast(                                                             \
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_tile, voff[q], (stage) * BK * 2, 0));      \
        } else {                                                                                          \
            const int64_t k0_ = (int64_t)(stage) * BK;                                                    \
            const int64_t kr_ = Kext - k0_ < BK ? Kext - k0_ : BK;                                        \
            const __amdgpu_buffer_rsrc_t rs_ = __builtin_amdgcn_make_buffer_rsrc(                         \
                (void*)(X0 + k0_ * s_k), (short)0,                                                        \
                kr_ > 0 && rows_valid > 0 ? (int)(((kr_ - 1) * s_k + rows_valid) * 2) : 0, 0x00020000);   \
            stg[set][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_, voff[q], 0, 0)); \
        }                                                                                                 \
    }
#define SG_WRITE1(set, q, slot)                                                                           \
    {                                                                                                     \
        const u32x4 w_ = KC ? stg[set][q] : sg_tr_row(stg[set], q);                                       \
        *reinterpret_cast<u32x4*>(lds + (slot) * STAGE + wofs[q]) = w_;                                   \
    }
#define SG_READ(slot, kk, f)                                                                              \
    {                                                                                                     \
        const uint16_t* L_ = lds + (slot) * STAGE;                                                        \
        const int c_ = (kk) * 2 + khalf;                                                                  \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) fa[f][i] =                                          \
            *reinterpret_cast<const bf16x8*>(L_ + a_base[i] + ((c_ ^ a_sw[i]) << 3));                     \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[f][j] =                                          \
            *reinterpret_cast<const bf16x8*>(L_ + b_base[j] + ((c_ ^ b_sw[j]) << 3));                     \
    }
// Iteration kt: phase A = MFMAs on (kt, first K half), reads of (kt, second half), LDS writes of
// stage kt+1 from staging set SET, then loads of the first half of stage kt+3 into SET (a transposed
// row needs all eight staged registers, so every write of the set precedes its first reload);
// barrier; phase B = MFMAs on (kt, second half), reads of (kt+1, first half), loads of the second
// half of stage kt+3.
#define SG_STEP(kt_, SET, DO_W, DO_L)                                                                     \
    {                                                                                                     \
        const int ktv = (kt_);                                                                            \
        const uint16_t* L1 = lds + (ktv & 1) * STAGE;                                                     \
        const int c1 = 2 + khalf;                                                                         \
        const int wslot = (ktv + 1) & 1;                                                                  \
        _Pragma("unroll") for (int st = 0; st < STEPS; ++st) {                                            \
            acc[st / TN][st % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][st % TN], fa[0][st / TN], \
                                                                            acc[st / TN][st % TN], 0, 0, 0); \
            if (st < TM) fa[1][st] = *reinterpret_cast<const bf16x8*>(L1 + a_base[st] + ((c1 ^ a_sw[st]) << 3)); \
            else if (st < TM + TN)                                                                        \
                fb[1][st - TM] =                                                                          \
                    *reinterpret_cast<const bf16x8*>(L1 + b_base[st - TM] + ((c1 ^ b_sw[st - TM]) << 3)); \
            if (st < NQ) {                                                                                \
                if (DO_W) SG_WRITE1(SET, st, wslot)                                                       \
            }                                                                                             \
            if (st >= NQ && st % 2 == 1) {                                                                \
                if (DO_L) SG_LOAD1(SET, (st - NQ) / 2, ktv + 3)                                           \
            }                                                                                             \
            __builtin_amdgcn_sched_barrier(0);                                                            \
        }                                                                                                 \
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                                 \
        __builtin_amdgcn_sched_barrier(0);                                                                \
        const uint16_t* L0 = lds + wslot * STAGE;                                                         \
        const int c0 = khalf;                                                                             \
        _Pragma("unroll") for (int st = 0; st < STEPS; ++st) {                                            \
            acc[st / TN][st % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][st % TN], fa[1][st / TN], \
                                                                            acc[st / TN][st % TN], 0, 0, 0); \
            if (st < TM) {                                                                                \
                if (DO_W) fa[0][st] = *reinterpret_cast<const bf16x8*>(L0 + a_base[st] + ((c0 ^ a_sw[st]) << 3)); \
            } else if (st < TM + TN) {                                                                    \
                if (DO_W)                                                                                 \
                    fb[0][st - TM] =                                                                      \
                        *reinterpret_cast<const bf16x8*>(L0 + b_base[st - TM] + ((c0 ^ b_sw[st - TM]) << 3)); \
            }                                                                                             \
            if (st % RSP == 1) {                                                                          \
                if (DO_L) SG_LOAD1(SET, RNH + st / RSP, ktv + 3)                                          \
            }                                                                                             \
            __builtin_amdgcn_sched_barrier(0);                                                            \
        }                                                                                                 \
    }

    // The pipeline, instantiated once per staging role (waves 0-1: operand A's layout, waves 2-3:
    // B's), so the pinned schedule has no layout branches. Both copies issue the same barriers.
    auto pipeline = [&](auto kc_tag) {
        constexpr bool KC = decltype(kc_tag)::value;
        // prologue: stage 0 -> set 0 -> slot 0; stage 1 -> set 1; stage 2 -> set 0
#pragma unroll
        for (int q = 0; q < NQ; ++q) SG_LOAD1(0, q, 0)
        if (nk > 1) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) SG_LOAD1(1, q, 1)
        }
        SG_WRITE1(0, 0, 0) SG_WRITE1(0, 1, 0) SG_WRITE1(0, 2, 0) SG_WRITE1(0, 3, 0)
        SG_WRITE1(0, 4, 0) SG_WRITE1(0, 5, 0) SG_WRITE1(0, 6, 0) SG_WRITE1(0, 7, 0)
        if (nk > 2) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) SG_LOAD1(0, q, 2)
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        SG_READ(0, 0, 0)
        int kt = 0;
        for (; kt + 4 < nk; kt += 2) {
            SG_STEP(kt, 1, true, true)
            SG_STEP(kt + 1, 0, true, true)
        }
        // tail (kt even; at most four iterations): plain order, static staging sets
#define SG_TAIL(j, SET)                                                                                   \
    if (kt + (j) < nk) {                                                                                  \
        const int ktv = kt + (j);                                                                         \
        const bool w = ktv + 1 < nk, l = ktv + 3 < nk;                                                    \
        SG_READ(ktv & 1, 1, 1)                                                                            \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) _Pragma("unroll") for (int jj = 0; jj < TN; ++jj)  \
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][jj], fa[0][i], acc[i][jj], 0, 0, 0); \
        if (w) {                                                                                          \
            SG_WRITE1(SET, 0, (ktv + 1) & 1) SG_WRITE1(SET, 1, (ktv + 1) & 1)                             \
            SG_WRITE1(SET, 2, (ktv + 1) & 1) SG_WRITE1(SET, 3, (ktv + 1) & 1)                             \
            SG_WRITE1(SET, 4, (ktv + 1) & 1) SG_WRITE1(SET, 5, (ktv + 1) & 1)                             \
            SG_WRITE1(SET, 6, (ktv + 1) & 1) SG_WRITE1(SET, 7, (ktv + 1) & 1)                             \
        }                                                                                                 \
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                                 \
        if (w) SG_READ((ktv + 1) & 1, 0, 0)                                                               \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) _Pragma("unroll") for (int jj = 0; jj < TN; ++jj)  \
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][jj], fa[1][i], acc[i][jj], 0, 0, 0); \
        if (l) {                                                                                          \
            _Pragma("unroll") for (int q = 0; q < NQ; ++q) SG_LOAD1(SET, q, ktv + 3)                      \
        }                                                                                                 \
    }
        SG_TAIL(0, 1)
        SG_TAIL(1, 0)
        SG_TAIL(2, 1)
        SG_TAIL(3, 0)
#undef SG_TAIL
    };
    if (nk > 0) {
        if (isA) pipeline(BoolTag<AK>{});
        else pipeline(BoolTag<BKC>{});
    }
#undef SG_LOAD1
#undef SG_WRITE1
#undef SG_READ
#undef SG_STEP
    // The MFMAs take the B fragment first, so a 32 x 32 accumulator holds an (n x m) block: a lane owns
    // row m = lane % 32 of C and, per group of four registers, 4 consecutive columns from
    // 8 q + 4 (lane / 32). Each lane stores 16 bytes (4 B per lane stored 4x the instructions: the
    // DeepSeek-shaped backward, whose weight gradients are 45 GB of fp32, 27.4 -> 25.4 ms).
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wn * 128 + j * 32 + 8 * q + 4 * khalf;
                const floatx4 val = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                if (m < M && n < p.N) *reinterpret_cast<floatx4*>(C + m * p.scm + n) = val;
            }
    }
}

// fp32 operands: one thread per output element, sequential fp32 FMA over K.
__global__ __launch_bounds__(256) void sg_gemm_f32_kernel(SgArgsF p) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t m_rel = blockIdx.y;
    const int g = blockIdx.z;
    if (n >= p.N || g >= p.G) return;
    int64_t M = p.M, kb = 0, ke = p.K, row_base = 0;
    if (p.mode == SG_ROWS) {
        row_base = p.offsets[p.e_begin + g];
        M = p.offsets[p.e_begin + g + 1] - row_base;
    } else if (p.mode == SG_KSPLIT) {
        kb = p.offsets[p.e_begin + g];
        ke = p.offsets[p.e_begin + g + 1];
    }
    const float* B = p.B + (int64_t)(p.mode == SG_ROWS ? g : 0) * p.b_group;
    float* C = p.C + (p.mode == SG_ROWS ? row_base * p.scm : (int64_t)g * p.c_group);
    for (int64_t m = m_rel; m < M; m += gridDim.y) {
        const float* A = p.A + (row_base + m) * p.sam;
        float acc = 0.f;
        for (int64_t k = kb; k < ke; ++k) acc = fmaf(A[k * p.sak], B[n * p.sbn + k * p.sbk], acc);
        C[m * p.scm + n] = acc;
    }
}

void launch_sg_gemm_bf16(const SgArgs& a, int64_t max_rows, hipStream_t s) {
    const int64_t tiles_n = (a.N + 255) / 256;
    int64_t blocks;
    if (a.mode == SG_ROWS) blocks = ((max_rows + 255) / 256 + a.G) * tiles_n;
    else blocks = ((a.M + 255) / 256) * tiles_n * a.G;
    if (blocks <= 0) return;
    const bool ak = a.sak == 1, bk = a.sbk == 1;
    if (ak && bk) sg_gemm_bf16_kernel<true, true><<<(unsigned)blocks, 256, 0, s>>>(a);
    else if (ak) sg_gemm_bf16_kernel<true, false><<<(unsigned)blocks, 256, 0, s>>>(a);
    else if (bk) sg_gemm_bf16_kernel<false, true><<<(unsigned)blocks, 256, 0, s>>>(a);
    else sg_gemm_bf16_kernel<false, false><<<(unsigned)blocks, 256, 0, s>>>(a);
}

void launch_sg_gemm_f32(const SgArgsF& a, int64_t max_rows, hipStream_t s) {
    const int64_t ymax = a.mode == SG_ROWS ? max_rows : a.M;
    const unsigned gy = (unsigned)(ymax < 1024 ? (ymax > 0 ? ymax : 1) : 1024);
    dim3 grid((unsigned)((a.N + 255) / 256), gy, (unsigned)a.G);
    sg_gemm_f32_kernel<<<grid, 256, 0, s>>>(a);
}

// ------------------------------------------------------------------------------------------------
// Elementwise and reduction kernels
// ------------------------------------------------------------------------------------------------

// Per token (one wave): dg[t, j] = <dy[t], y_perm[row]> and dYp[row] = g[t, j] * dy[t] for each kept
// slot (row = inv_pos[t*k + j] >= 0); dropped slots get dg = 0 and no row.
template <bool BF16, int KMAX>
__global__ __launch_bounds__(256) void bwd_combine_kernel(const void* __restrict__ dy, const void* __restrict__ y_perm,
                                                          const int32_t* __restrict__ inv_pos,
                                                          const float* __restrict__ topk_w, int64_t T, int d, int k,
                                                          float* __restrict__ dg, void* __restrict__ dYp) {
    constexpr int EB = BF16 ? 2 : 4, EPV = 16 / EB;  // element bytes, elements per 16-byte vector
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int mypos = lane < k ? inv_pos[t * k + lane] : -1;
    const float myg = lane < k ? topk_w[t * k + lane] : 0.f;
    const int64_t row_bytes = (int64_t)d * EB;
    const uint8_t* dyr = static_cast<const uint8_t*>(dy) + t * row_bytes;
    const uint8_t* yp = static_cast<const uint8_t*>(y_perm);
    uint8_t* dyp = static_cast<uint8_t*>(dYp);
    float dot[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) dot[j] = 0.f;
    const int nvec = d / EPV;
    for (int c0 = lane; c0 < nvec; c0 += 64) {
        float f[EPV];
        const u32x4 dv = ld16(dyr + (int64_t)c0 * 16);
        if (BF16) unpack8(dv, f);
        else
#pragma unroll
            for (int i = 0; i < EPV; ++i) f[i] = __uint_as_float(dv[i]);
        u32x4 yv[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int p = j < k ? __builtin_amdgcn_readlane(mypos, j) : -1;
            if (p >= 0) yv[j] = ld16(yp + (int64_t)p * row_bytes + (int64_t)c0 * 16);
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int p = j < k ? __builtin_amdgcn_readlane(mypos, j) : -1;
            if (p < 0) continue;
            const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myg), j));
            float yf[EPV], o[EPV];
            if (BF16) unpack8(yv[j], yf);
            else
#pragma unroll
                for (int i = 0; i < EPV; ++i) yf[i] = __uint_as_float(yv[j][i]);
#pragma unroll
            for (int i = 0; i < EPV; ++i) {
                dot[j] = fmaf(f[i], yf[i], dot[j]);
                o[i] = g * f[i];
            }
            u32x4 ov;
            if (BF16) ov = pack8(o);
            else
#pragma unroll
                for (int i = 0; i < EPV; ++i) ov[i] = __float_as_uint(o[i]);
            st16(dyp + (int64_t)p * row_bytes + (int64_t)c0 * 16, ov);
        }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
            const int p = __builtin_amdgcn_readlane(mypos, j);
            const float s = wave_sum(dot[j]);
            if (lane == 0) dg[t * k + j] = p < 0 ? 0.f : s;
        }
    }
}

// h = act(pre) on n_rows rows: SwiGLU pre = [a | u] (2F wide) -> silu(a) * u; GELU pre = z -> gelu(z).
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_act_fwd_kernel(const void* __restrict__ pre, int64_t n_rows, int F, int act,
                                                          void* __restrict__ h) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_rows * F) return;
    const int64_t r = i / F;
    const int f = (int)(i - r * F);
    float v;
    if (act == MOE_SWIGLU) v = silu_b(ld_elem<BF16>(pre, r * 2 * F + f)) * ld_elem<BF16>(pre, r * 2 * F + F + f);
    else v = gelu_b(ld_elem<BF16>(pre, r * F + f));
    st_elem<BF16>(h, i, v);
}

// dAU from dh (fp32) and the pre-activations: SwiGLU da = dh * u * silu'(a), du = dh * silu(a);
// GELU dz = dh * gelu'(z).
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_act_bwd_kernel(const float* __restrict__ dh, const void* __restrict__ pre,
                                                          int64_t n_rows, int F, int act, void* __restrict__ dAU) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_rows * F) return;
    const int64_t r = i / F;
    const int f = (int)(i - r * F);
    const float g = dh[i];
    if (act == MOE_SWIGLU) {
        const float a = ld_elem<BF16>(pre, r * 2 * F + f), u = ld_elem<BF16>(pre, r * 2 * F + F + f);
        st_elem<BF16>(dAU, r * 2 * F + f, g * u * silu_grad_b(a));
        st_elem<BF16>(dAU, r * 2 * F + F + f, g * silu_b(a));
    } else {
        st_elem<BF16>(dAU, i, g * gelu_grad_b(ld_elem<BF16>(pre, i)));
    }
}

// dx32[t] = sum over kept slots of dXp[inv_pos[t*k + j]] (+ extra[t]), fp32, in slot order.
template <int KMAX>
__global__ __launch_bounds__(256) void bwd_unpermute_kernel(const float* __restrict__ dXp,
                                                            const int32_t* __restrict__ inv_pos,
                                                            const float* __restrict__ extra, int64_t T, int d, int k,
                                                            float* __restrict__ dx32) {
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int mypos = lane < k ? inv_pos[t * k + lane] : -1;
    const int nvec = d / 4;
    for (int c0 = lane; c0 < nvec; c0 += 64) {
        floatx4 v[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int p = j < k ? __builtin_amdgcn_readlane(mypos, j) : -1;
            if (p >= 0) v[j] = *reinterpret_cast<const floatx4*>(dXp + (int64_t)p * d + (int64_t)c0 * 4);
        }
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int p = j < k ? __builtin_amdgcn_readlane(mypos, j) : -1;
            if (p < 0) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += v[j][i];
        }
        if (extra != nullptr) {
            const floatx4 xe = *reinterpret_cast<const floatx4*>(extra + t * d + (int64_t)c0 * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += xe[i];
        }
        *reinterpret_cast<floatx4*>(dx32 + t * d + (int64_t)c0 * 4) = floatx4{acc[0], acc[1], acc[2], acc[3]};
    }
}

// Column sums per group: out[g][c] = sum over rows r in [offsets[g], offsets[g+1]) of src[r][c],
// rows in ascending order (fixed order, so deterministic).
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_colsum_kernel(const void* __restrict__ src, const int32_t* __restrict__ offsets,
                                                         int e_begin, int ncols, float* __restrict__ out) {
    const int g = blockIdx.y;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= ncols) return;
    const int r0 = offsets[e_begin + g], r1 = offsets[e_begin + g + 1];
    float acc = 0.f;
    for (int r = r0; r < r1; ++r) acc += ld_elem<BF16>(src, (int64_t)r * ncols + c);
    out[(int64_t)g * ncols + c] = acc;
}

// Router logit gradient per token (one wave): the gate backward for the scoring in use, plus the
// balancing term coef * E * sum f P with f = counts / T held constant.
template <int EPL>
__global__ __launch_bounds__(256) void bwd_gate_kernel(const float* __restrict__ logits,
                                                       const int32_t* __restrict__ topk_idx,
                                                       const float* __restrict__ dg, const int32_t* __restrict__ counts,
                                                       float aux_coef, int64_t T, int E, int k, int score, int renorm,
                                                       float* __restrict__ dl) {
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const float* lt = logits + t * E;
    float l[EPL], out[EPL];
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        l[i] = e < E ? lt[e] : -INFINITY;
        out[i] = 0.f;
        lmax = fmaxf(lmax, l[i]);
    }
    const bool softmax = score == MOE_SOFTMAX;
    // lane j < k holds slot j: its expert, logit and gate gradient
    const int ej = lane < k ? topk_idx[t * k + lane] : -1;
    const float dgj = lane < k ? dg[t * k + lane] : 0.f;
    float lj = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        // the logit of expert ej is held by lane ej % 64, register ej / 64
        const int src = ej >= 0 ? (ej & 63) : 0;
        const float v = __shfl(l[i], src, 64);
        if (ej >= 0 && (ej >> 6) == i) lj = v;
    }
    if (softmax && !renorm) {
        // dl = p * (dp - <p, dp>), dp = dg at the selected experts
        const float m = wave_max(lmax);
        float z = 0.f, p[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            p[i] = lane + 64 * i < E ? expf(l[i] - m) : 0.f;
            z += p[i];
        }
        const float invZ = 1.0f / wave_sum(z);
        float dpsum = 0.f;  // <p, dp> over the selection, formed on the slot lanes
        const float pj = lane < k ? expf(lj - m) * invZ : 0.f;
        dpsum = wave_sum(pj * dgj);
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            float dp = 0.f;
            for (int j = 0; j < k; ++j) {
                const int ejj = __shfl(ej, j, 64);
                const float dgg = __shfl(dgj, j, 64);
                if (ejj == e) dp = dgg;
            }
            out[i] = p[i] * invZ * (dp - dpsum);
        }
    } else {
        // selected slots only: softmax over the selected logits, or sigmoid normalised over them
        float gsel, dsel;
        if (softmax) {
            const float ms = wave_max(lane < k ? lj : -INFINITY);
            const float ex = lane < k ? expf(lj - ms) : 0.f;
            gsel = ex / wave_sum(ex);
            const float c = wave_sum(lane < k ? gsel * dgj : 0.f);
            dsel = gsel * (dgj - c);
        } else {
            const float s = lane < k ? sigm(lj) : 0.f;
            const float Z = wave_sum(s);
            gsel = s / Z;
            const float c = wave_sum(lane < k ? gsel * dgj : 0.f);
            dsel = (dgj - c) / Z * s * (1.0f - s);
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            for (int j = 0; j < k; ++j) {
                const int ejj = __shfl(ej, j, 64);
                const float v = __shfl(dsel, j, 64);
                if (ejj == e) out[i] = v;
            }
        }
    }
    if (aux_coef != 0.f) {
        // p = balance distribution; dl += p' * (dp - <p, dp>) with dp_e = coef * E * f_e / T
        const float m = wave_max(lmax);
        float q[EPL], s[EPL], z = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            s[i] = e < E ? (softmax ? expf(l[i] - m) : sigm(l[i])) : 0.f;
            z += s[i];
        }
        const float Z = wave_sum(z);
        float pdp = 0.f, dpv[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            q[i] = s[i] / Z;
            dpv[i] = e < E ? aux_coef * (float)E * ((float)counts[e] / (float)T) / (float)T : 0.f;
            pdp += q[i] * dpv[i];
        }
        pdp = wave_sum(pdp);
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const float c = dpv[i] - pdp;
            out[i] += softmax ? q[i] * c : c / Z * s[i] * (1.0f - s[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) dl[t * E + e] = out[i];
    }
}

// dW_r[e][c] = sum_t dl[t][e] x[t][c]. Block (column block, 8 experts, token chunk z) sums its
// kRouterChunk tokens in order into partials[z][e][c]; bwd_router_reduce adds the chunks in order.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_router_wgrad_kernel(const float* __restrict__ dl, const void* __restrict__ x,
                                                               int64_t T, int E, int d, float* __restrict__ partials) {
    constexpr int EB = kRouterWgradExperts;
    __shared__ float s_dl[kRouterChunk][EB];  // dl of the chunk's tokens for this block's experts
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int e0 = blockIdx.y * EB;
    const int64_t t0 = (int64_t)blockIdx.z * kRouterChunk;
    const int64_t t1 = t0 + kRouterChunk < T ? t0 + kRouterChunk : T;
    const int ne = E - e0 < EB ? E - e0 : EB;
    for (int i = threadIdx.x; i < kRouterChunk * EB; i += 256) {
        const int tt = i / EB, j = i % EB;
        s_dl[tt][j] = (t0 + tt < t1 && j < ne) ? dl[(t0 + tt) * E + e0 + j] : 0.f;
    }
    __syncthreads();
    if (c >= d) return;
    float acc[EB];
#pragma unroll
    for (int i = 0; i < EB; ++i) acc[i] = 0.f;
    const int n = (int)(t1 - t0);
    int tt = 0;
    for (; tt + 4 <= n; tt += 4) {  // four token rows in flight
        float xv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[u] = ld_elem<BF16>(x, (t0 + tt + u) * d + c);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < EB; ++i) acc[i] = fmaf(s_dl[tt + u][i], xv[u], acc[i]);
    }
    for (; tt < n; ++tt) {
        const float xv = ld_elem<BF16>(x, (t0 + tt) * d + c);
#pragma unroll
        for (int i = 0; i < EB; ++i) acc[i] = fmaf(s_dl[tt][i], xv, acc[i]);
    }
    float* out = partials + (int64_t)blockIdx.z * E * d;
#pragma unroll
    for (int i = 0; i < EB; ++i)
        if (i < ne) out[(int64_t)(e0 + i) * d + c] = acc[i];
}

__global__ __launch_bounds__(256) void bwd_router_reduce_kernel(const float* __restrict__ partials, int nchunks,
                                                                int64_t n, float* __restrict__ dw_r) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = 0.f;
    for (int z = 0; z < nchunks; ++z) acc += partials[(int64_t)z * n + i];
    dw_r[i] = acc;
}

// dx[t][c] = dx32[t][c] + sum_e dl[t][e] W_r[e][c], written in the layer dtype (one rounding).
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_router_dgrad_kernel(const float* __restrict__ dx32,
                                                               const float* __restrict__ dl,
                                                               const float* __restrict__ w_r, int64_t T, int E, int d,
                                                               void* __restrict__ dx) {
    constexpr int TB = kRouterDgradTokens, EC = 256;
    __shared__ float s_dl[TB][EC];  // dl of the block's tokens, one chunk of experts at a time
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * TB;
    const int nt = T - t0 < TB ? (int)(T - t0) : TB;
    const bool col = c < d;
    float acc[TB];
#pragma unroll
    for (int q = 0; q < TB; ++q) acc[q] = (col && q < nt) ? dx32[(t0 + q) * d + c] : 0.f;
    for (int e0 = 0; e0 < E; e0 += EC) {
        const int ne = E - e0 < EC ? E - e0 : EC;
        __syncthreads();
        for (int i = threadIdx.x; i < TB * EC; i += 256) {
            const int q = i / EC, j = i % EC;
            s_dl[q][j] = (q < nt && j < ne) ? dl[(t0 + q) * E + e0 + j] : 0.f;
        }
        __syncthreads();
        if (!col) continue;
        int j = 0;
        for (; j + 4 <= ne; j += 4) {  // four router rows in flight
            float wv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) wv[u] = w_r[(int64_t)(e0 + j + u) * d + c];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int q = 0; q < TB; ++q) acc[q] = fmaf(s_dl[q][j + u], wv[u], acc[q]);
        }
        for (; j < ne; ++j) {
            const float wv = w_r[(int64_t)(e0 + j) * d + c];
#pragma unroll
            for (int q = 0; q < TB; ++q) acc[q] = fmaf(s_dl[q][j], wv, acc[q]);
        }
    }
    if (!col) return;
#pragma unroll
    for (int q = 0; q < TB; ++q)
        if (q < nt) st_elem<BF16>(dx, (t0 + q) * d + c, acc[q]);
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

void launch_bwd_combine(int dtype, const void* dy, const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                        int64_t T, int d, int k, float* dg, void* dYp, hipStream_t s) {
    const unsigned nb = (unsigned)((T + 3) / 4);
#define MOE_BWD_COMBINE(B_, K_) bwd_combine_kernel<B_, K_><<<nb, 256, 0, s>>>(dy, y_perm, inv_pos, topk_w, T, d, k, dg, dYp)
    if (dtype == MOE_BF16) {
        if (k <= 2) MOE_BWD_COMBINE(true, 2);
        else if (k <= 4) MOE_BWD_COMBINE(true, 4);
        else if (k <= 8) MOE_BWD_COMBINE(true, 8);
        else if (k <= 16) MOE_BWD_COMBINE(true, 16);
        else MOE_BWD_COMBINE(true, 32);
    } else {
        if (k <= 2) MOE_BWD_COMBINE(false, 2);
        else if (k <= 4) MOE_BWD_COMBINE(false, 4);
        else if (k <= 8) MOE_BWD_COMBINE(false, 8);
        else if (k <= 16) MOE_BWD_COMBINE(false, 16);
        else MOE_BWD_COMBINE(false, 32);
    }
#undef MOE_BWD_COMBINE
}

void launch_bwd_act_fwd(int dtype, const void* pre, int64_t n_rows, int F, int act, void* h, hipStream_t s) {
    if (n_rows <= 0) return;
    if (dtype == MOE_BF16) bwd_act_fwd_kernel<true><<<blocks_for(n_rows * F), 256, 0, s>>>(pre, n_rows, F, act, h);
    else bwd_act_fwd_kernel<false><<<blocks_for(n_rows * F), 256, 0, s>>>(pre, n_rows, F, act, h);
}

// Batched bf16 transpose: src [G][R][C] -> dst [G][C][R] (R, C multiples of 64), 64 x 64 tiles
// through LDS: 16-byte loads along C, 16-byte stores along R.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                                             uint16_t* __restrict__ dst) {
    __shared__ uint16_t tile[64][64 + 2];
    const int64_t g = blockIdx.z;
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const uint16_t* sg = src + g * R * C;
    uint16_t* dg = dst + g * R * C;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int v = it * 256 + threadIdx.x;  // 512 vectors of 8 elements
        const int r = v >> 3, c = (v & 7) * 8;
        const u32x4 q = ld16(sg + (r0 + r) * C + c0 + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tile[r][c + 2 * i] = (uint16_t)(q[i] & 0xffffu);
            tile[r][c + 2 * i + 1] = (uint16_t)(q[i] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int v = it * 256 + threadIdx.x;
        const int c = v >> 3, r = (v & 7) * 8;  // output row c (a source column), 8 source rows
        u32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (uint32_t)tile[r + 2 * i][c] | ((uint32_t)tile[r + 2 * i + 1][c] << 16);
        st16(dg + (c0 + c) * R + r0 + r, q);
    }
}

// Weight gradients on the wide GEMM's K-grouped mode: expert e's rows of a permuted buffer become
// columns [poff[e], poff[e] + rows_e) of a transposed copy, zero-padded to the next multiple of 64
// (64 columns for an expert without rows, so every expert has at least one stage). poff[E] is the
// padded total; blk[j] is the expert owning 64-column block j, or -1 past it (j < nblk).
__global__ __launch_bounds__(256) void wgrad_pad_offsets_kernel(const int32_t* __restrict__ offsets, int E, int nblk,
                                                               int32_t* __restrict__ poff, int32_t* __restrict__ blk) {
    __shared__ int s_poff[1025];
    if (threadIdx.x == 0) {  // E <= 1024 additions in expert order
        int acc = 0;
        for (int e = 0; e < E; ++e) {
            s_poff[e] = acc;
            const int rows = offsets[e + 1] - offsets[e];
            acc += rows > 0 ? (rows + 63) / 64 * 64 : 64;
        }
        s_poff[E] = acc;
    }
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += 256) poff[e] = s_poff[e];
    for (int j = threadIdx.x; j < nblk; j += 256) {
        const int c = j * 64;
        int owner = -1;
        if (c < s_poff[E]) {  // the last expert whose range starts at or before c
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_poff[mid] <= c) lo = mid;
                else hi = mid - 1;
            }
            owner = lo;
        }
        blk[j] = owner;
    }
}

// dst[c][poff[e] + i] = src[offsets[e] + i][c] for the rows i of expert e, zero in the padding: 64 x 64
// tiles through LDS, block (x, y) covering source columns 64 x and destination columns 64 y (one
// expert's, as every padded range is a multiple of 64). C is a multiple of 64; dst rows are ld long.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ src, int64_t C,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ poff,
                                                            const int32_t* __restrict__ blk, int64_t ld,
                                                            uint16_t* __restrict__ dst) {
    __shared__ uint16_t tile[64][64 + 2];
    const int e = blk[blockIdx.y];
    if (e < 0) return;  // uniform per block
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int j0 = (int)blockIdx.y * 64;
    const int i0 = j0 - poff[e], rows = offsets[e + 1] - offsets[e];
    const int64_t r0 = (int64_t)offsets[e] + i0;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int v = it * 256 + threadIdx.x;  // 512 vectors of 8 elements
        const int r = v >> 3, c = (v & 7) * 8;
        u32x4 q = {0u, 0u, 0u, 0u};
        if (i0 + r < rows) q = ld16(src + (r0 + r) * C + c0 + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tile[r][c + 2 * i] = (uint16_t)(q[i] & 0xffffu);
            tile[r][c + 2 * i + 1] = (uint16_t)(q[i] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int v = it * 256 + threadIdx.x;
        const int c = v >> 3, r = (v & 7) * 8;  // destination row c0 + c, 8 destination columns
        u32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (uint32_t)tile[r + 2 * i][c] | ((uint32_t)tile[r + 2 * i + 1][c] << 16);
        st16(dst + (c0 + c) * ld + j0 + r, q);
    }
}

void launch_wgrad_pad_offsets(const int32_t* offsets, int E, int nblk, int32_t* poff, int32_t* blk, hipStream_t s) {
    wgrad_pad_offsets_kernel<<<1, 256, 0, s>>>(offsets, E, nblk, poff, blk);
}

void launch_transpose_pad(const void* src, int64_t C, const int32_t* offsets, const int32_t* poff,
                          const int32_t* blk, int nblk, int64_t ld, void* dst, hipStream_t s) {
    dim3 grid((unsigned)(C / 64), (unsigned)nblk);
    transpose_pad_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src), C, offsets, poff, blk, ld,
                                              static_cast<uint16_t*>(dst));
}

void launch_transpose_bf16(const void* src, int64_t G, int64_t R, int64_t C, void* dst, hipStream_t s) {
    dim3 grid((unsigned)(C / 64), (unsigned)(R / 64), (unsigned)G);
    transpose_bf16_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src), R, C, static_cast<uint16_t*>(dst));
}

void launch_bwd_act_bwd(int dtype, const float* dh, const void* pre, int64_t n_rows, int F, int act, void* dAU,
                        hipStream_t s) {
    if (n_rows <= 0) return;
    if (dtype == MOE_BF16) bwd_act_bwd_kernel<true><<<blocks_for(n_rows * F), 256, 0, s>>>(dh, pre, n_rows, F, act, dAU);
    else bwd_act_bwd_kernel<false><<<blocks_for(n_rows * F), 256, 0, s>>>(dh, pre, n_rows, F, act, dAU);
}

void launch_bwd_unpermute(const float* dXp, const int32_t* inv_pos, const float* extra, int64_t T, int d, int k,
                          float* dx32, hipStream_t s) {
    const unsigned nb = (unsigned)((T + 3) / 4);
    if (k <= 2) bwd_unpermute_kernel<2><<<nb, 256, 0, s>>>(dXp, inv_pos, extra, T, d, k, dx32);
    else if (k <= 4) bwd_unpermute_kernel<4><<<nb, 256, 0, s>>>(dXp, inv_pos, extra, T, d, k, dx32);
    else if (k <= 8) bwd_unpermute_kernel<8><<<nb, 256, 0, s>>>(dXp, inv_pos, extra, T, d, k, dx32);
    else if (k <= 16) bwd_unpermute_kernel<16><<<nb, 256, 0, s>>>(dXp, inv_pos, extra, T, d, k, dx32);
    else bwd_unpermute_kernel<32><<<nb, 256, 0, s>>>(dXp, inv_pos, extra, T, d, k, dx32);
}

void launch_bwd_colsum(int dtype, const void* src, const int32_t* offsets, int e_begin, int G, int ncols, float* out,
                       hipStream_t s) {
    dim3 grid(blocks_for(ncols), (unsigned)G);
    if (dtype == MOE_BF16) bwd_colsum_kernel<true><<<grid, 256, 0, s>>>(src, offsets, e_begin, ncols, out);
    else bwd_colsum_kernel<false><<<grid, 256, 0, s>>>(src, offsets, e_begin, ncols, out);
}

void launch_bwd_gate(const float* logits, const int32_t* topk_idx, const float* dg, const int32_t* counts,
                     float aux_coef, int64_t T, int E, int k, int score, int renorm, float* dl, hipStream_t s) {
    const unsigned nb = (unsigned)((T + 3) / 4);
#define MOE_GATE(EPL) bwd_gate_kernel<EPL><<<nb, 256, 0, s>>>(logits, topk_idx, dg, counts, aux_coef, T, E, k, score, renorm, dl)
    if (E <= 64) MOE_GATE(1);
    else if (E <= 128) MOE_GATE(2);
    else if (E <= 256) MOE_GATE(4);
    else if (E <= 512) MOE_GATE(8);
    else MOE_GATE(16);
#undef MOE_GATE
}

size_t bwd_router_partials_bytes(int64_t T, int E, int d) {
    return (size_t)((T + kRouterChunk - 1) / kRouterChunk) * E * d * sizeof(float);
}

void launch_bwd_router(int dtype, const float* dl, const void* x, const float* w_r, const float* dx32, int64_t T,
                       int E, int d, float* partials, float* dw_r, void* dx, hipStream_t s) {
    const int nchunks = (int)((T + kRouterChunk - 1) / kRouterChunk);
    const unsigned cblk = (unsigned)((d + 255) / 256);
    dim3 gw(cblk, (unsigned)((E + kRouterWgradExperts - 1) / kRouterWgradExperts), (unsigned)nchunks);
    dim3 gd(cblk, (unsigned)((T + kRouterDgradTokens - 1) / kRouterDgradTokens));
    const int64_t n = (int64_t)E * d;
    if (dtype == MOE_BF16) {
        bwd_router_wgrad_kernel<true><<<gw, 256, 0, s>>>(dl, x, T, E, d, partials);
        bwd_router_dgrad_kernel<true><<<gd, 256, 0, s>>>(dx32, dl, w_r, T, E, d, dx);
    } else {
        bwd_router_wgrad_kernel<false><<<gw, 256, 0, s>>>(dl, x, T, E, d, partials);
        bwd_router_dgrad_kernel<false><<<gd, 256, 0, s>>>(dx32, dl, w_r, T, E, d, dx);
    }
    bwd_router_reduce_kernel<<<blocks_for(n), 256, 0, s>>>(partials, nchunks, n, dw_r);
}

}  // namespace moe

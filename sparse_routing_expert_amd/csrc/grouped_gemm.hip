// moe_expert_up / moe_expert_down / moe_shared_ffn kernels: all experts' FFN products as one grouped
// GEMM launch per projection ("Router Optimization Techniques", Production Deployment 1 and What
// Most Articles Miss 2: one grouped-GEMM kernel over a contiguous token workspace instead of one
// kernel per expert). The expert FFNs are SwiGLU ((SiLU(x Wg^T) * x Wu^T) Wd^T; same page, What Is
// It?) or Linear + GELU + Linear with biases ("Fine-tuning and serving MoE models").
//
// Tile schedule: every block turns the device-side expert offsets into a prefix sum of per-expert
// row-tile counts in LDS (the host never reads the offsets, so there is no synchronisation). The
// grid is an upper bound; a block decodes its id into (expert, row tile, column tile) and exits
// when it is past the end, so empty experts own no tile and a ragged last tile is masked, not
// padded. Blocks are dealt round-robin to the 8 XCDs (block i runs on XCD i % 8), so the decode
// hands each XCD a contiguous chunk of an expert-major tile sequence in which groups of GM row
// tiles sweep the column panels: the row tiles that share a weight panel run on the same XCD and
// read it through that XCD's L2 once.
//
// bf16 kernels (one launch per projection, plus a short fixup launch when the last round of tiles is
// split along K):
//  - gemm_bf16_persistent_kernel: one block of eight waves per CU walks 256 x 256 output tiles
//    (SwiGLU: 128 gate and the matching 128 up columns, so a lane holds gate and up of the same
//    output element) in an XCD-aware order; two groups of four waves alternate LDS fragment reads
//    and MFMA clusters (ping-pong), and the LDS ring runs on across tiles.
//  - gemm_bf16_wide_kernel, for expert groups averaging at least 2048 rows: 256 x 384 tiles (SwiGLU:
//    192 gate and the matching 192 up columns), or 256 x 256 past 128 groups, in the same order;
//    four waves that place their memory instructions between their own MFMAs, and 64-wide K
//    stages, so each DMA reads whole 128-byte row pieces. Its K-grouped mode (KgArgs) computes the
//    backward's weight gradients, one product per expert over that expert's range of K.
//  - gemm_bf16_kernel: four waves on one 64 x 128 (or 64 x 64) tile with a 6- (8-) stage ring, two
//    blocks per CU, for groups of a few dozen rows (decode batches), whose time is spent streaming
//    the weight panels.
// All use v_mfma_f32_32x32x16_bf16 with fp32 accumulators. Operands stream into an LDS ring with
// buffer_load ... lds (global -> LDS without registers); buffer descriptors bound each tile's rows,
// so rows past an expert's end or columns past n_out read as zero and nothing is clamped. LDS rows of
// 64 bytes have their four 16-byte chunks XOR-swizzled by (row >> 2) & 3, rows of 128 bytes their
// eight chunks by (row >> 1) & 7, which keeps the 128-bit operand reads on gfx950 free of bank
// conflicts (16 lanes per LDS cycle, 64 banks). Waits on the DMA are explicit (vmcnt), because the
// compiler cannot see it.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe.h"

namespace moe {

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float gelu_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

struct TileCoord {
    int64_t row0, row_end;  // rows [row0, min(row0 + BM, row_end)) of A and C
    int e;                  // weight group
    int n0;                 // first output column
    bool valid;
};

// s_ts[g] = sum over groups g' < g of ceil(rows_g' / BM); s_ts[n_groups] = total (n_groups <= 1024).
// Needs a block of NT threads (256 or 512); each thread owns up to 1024 / NT consecutive groups.
template <int BM, int NT>
__device__ __forceinline__ void build_schedule(const int32_t* __restrict__ offsets, int e_begin, int n_groups,
                                               int* s_ts, int* s_wave) {
    constexpr int GPT = 1024 / NT;
    static_assert(NT * GPT == 1024 && NT % 64 == 0, "schedule block");
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    int n[GPT], sum = 0;
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int g = tid * GPT + i;
        n[i] = 0;
        if (g < n_groups) {
            const int rows = offsets[e_begin + g + 1] - offsets[e_begin + g];
            n[i] = (rows + BM - 1) / BM;
        }
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
    for (int i = 0; i < GPT; ++i) {
        const int g = tid * GPT + i;
        if (g < n_groups) s_ts[g] = base;
        base += n[i];
    }
    if (tid == NT - 1) s_ts[n_groups] = base;
    __syncthreads();
}

// Block id -> tile: XCD-contiguous chunks of an expert-major sequence; inside an expert, groups of
// GM row tiles sweep the column tiles (row tile fastest).
template <int BM, int BNO, int GM>
__device__ __forceinline__ TileCoord decode_tile(const int32_t* __restrict__ offsets, const int* s_ts,
                                                 int e_begin, int n_groups, int64_t dense_rows, int n_out) {
    TileCoord tc;
    const int n_tiles_n = (n_out + BNO - 1) / BNO;
    const int64_t m_tiles = offsets ? (int64_t)s_ts[n_groups] : (dense_rows + BM - 1) / BM;
    const int64_t R = m_tiles * n_tiles_n;
    const int64_t per = (R + 7) / 8;
    const int64_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int64_t lin = xcd * per + slot;
    tc.valid = slot < per && lin < R;
    if (!tc.valid) return tc;
    int g = 0;
    int64_t g_mt = m_tiles, local = lin;
    if (offsets) {
        const int64_t key = lin / n_tiles_n;  // group g owns [s_ts[g] * NT, s_ts[g + 1] * NT)
        int lo = 0, hi = n_groups - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_ts[mid] <= key) lo = mid;
            else hi = mid - 1;
        }
        g = lo;
        g_mt = s_ts[g + 1] - s_ts[g];
        local = lin - (int64_t)s_ts[g] * n_tiles_n;
    }
    const int64_t grp = local / ((int64_t)GM * n_tiles_n);
    const int64_t first_m = grp * GM;
    const int64_t gsz = g_mt - first_m < GM ? g_mt - first_m : GM;
    const int64_t rem = local - grp * GM * n_tiles_n;
    const int64_t mt = first_m + rem % gsz;  // row tile within the group
    tc.n0 = (int)(rem / gsz) * BNO;
    if (offsets) {
        tc.e = e_begin + g;
        tc.row0 = offsets[tc.e] + mt * BM;
        tc.row_end = offsets[tc.e + 1];
    } else {
        tc.e = 0;
        tc.row0 = mt * BM;
        tc.row_end = dense_rows;
    }
    return tc;
}

// Raw buffer resource (gfx9 layout): base, stride 0, byte range; word 3 = 0x00020000.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from the buffer (byte offset voff + soff) into LDS at m0 + 16 * lane. Written as
// inline asm so the compiler's conservative wait-before-every-LDS-read for LDS DMA does not apply;
// the waits are placed explicitly with wait_vm. No register is written by the instruction.
__device__ __forceinline__ void dma16(uint32_t m0, int voff, i32x4 rsrc, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// wait until at most n stages of NQ DMA instructions each are in flight (0 <= n <= 6)
template <int NQ>
__device__ __forceinline__ void wait_stages(int n) {
    if (n <= 0) wait_vm<0>();
    else if (n == 1) wait_vm<NQ>();
    else if (n == 2) wait_vm<2 * NQ>();
    else if (n == 3) wait_vm<3 * NQ>();
    else if (n == 4) wait_vm<4 * NQ>();
    else if (n == 5) wait_vm<5 * NQ>();
    else wait_vm<6 * NQ>();
}
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }  // 128-byte rows (wide kernel)
// Byte offset of 16-byte chunk c of row R of a gathered tile (rows row0 + R of the group are tokens
// gather[row0 + R] of A). The descriptor spans A, which the host keeps below 2 GB; rows past the
// group's end get an offset of 2 GB, out of the descriptor's range at every K stage, so they read as
// zeros without a memory request (reading the group's last row instead cost a small group's tile as
// many L2 requests again as its own rows: 128-row groups in 256-row tiles).
constexpr uint32_t kGatherPastEnd = 0x80000000u;
__device__ __forceinline__ int gathered_voff(const int32_t* __restrict__ gather, int64_t row0, int64_t row_end, int R,
                                             int K, int c) {
    if (row0 + R >= row_end) return (int)kGatherPastEnd;
    return (int)((uint32_t)gather[row0 + R] * (uint32_t)(K * 2) + (uint32_t)(c * 16));
}
// The same for the RPD rows r0 + [0, RPD) of one DMA instruction (64 / RPD lanes per row, r0 and the
// tile wave-uniform; chunk c of row R at position c ^ swz(R) for 64-byte rows, c ^ swz8(R) for
// 128-byte rows), read with scalar loads: the persistent kernels call this while their own LDS-DMA
// loads are in flight, and a vector load here would make the wave wait for all of those before it
// could use the index. The gather buffer holds at least 256 entries past its last row, so the RPD
// reads stay inside it when the group ends within them. The lane id is recomputed here rather than
// kept from the kernel's start, so the per-DMA chunk offsets need no registers (or spill slots)
// across the main loop.
__device__ __forceinline__ int lane_here() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
template <int RPD>
__device__ __forceinline__ int gathered_voff_uniform(const int32_t* __restrict__ gather, int64_t row0,
                                                     int64_t row_end, int r0, int K) {
    constexpr int LPR = 64 / RPD;  // lanes per row
    const int lane = lane_here();
    const int R = r0 + lane / LPR;
    const int c = (lane & (LPR - 1)) ^ (RPD == 16 ? swz(R) : swz8(R));
    const int64_t base = ((int64_t)__builtin_amdgcn_readfirstlane((int)(row0 >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)row0);
    // constant address space + readfirstlane: uniform loads the compiler must not fold into one
    // per-lane vector load
    typedef const __attribute__((address_space(4))) int32_t* cptr;
    const cptr g = (cptr)(gather + base + __builtin_amdgcn_readfirstlane(r0));
    const int i = lane / LPR;
    int v = __builtin_amdgcn_readfirstlane(g[0]);
#pragma unroll
    for (int t = 1; t < RPD; ++t) {
        const int gt = __builtin_amdgcn_readfirstlane(g[t]);
        v = i == t ? gt : v;
    }
    // rows left in the group from the tile start, in 32 bits (a tile spans at most 256 rows)
    const int64_t left64 = row_end - row0;
    const int left = __builtin_amdgcn_readfirstlane(left64 > 4096 ? 4096 : (int)left64);
    if (r0 + i >= left) return (int)kGatherPastEnd;
    return (int)((uint32_t)v * (uint32_t)(K * 2) + (uint32_t)(c * 16));
}

}  // namespace

template <int BM, int BN, int EPI, int NS, int GM, bool KT>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ B,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ C,
                                                           const int32_t* __restrict__ offsets, int e_begin,
                                                           int n_groups, int64_t dense_rows, int n_out, int K,
                                                           const int32_t* __restrict__ gather, uint32_t a_bytes) {
    constexpr int BK = 32, WM = 2, WN = 2;
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int WTM = BM / WM, TM = WTM / 32;
    constexpr int BNO = GATED ? BN / 2 : BN, WTNO = BNO / WN, TNO = WTNO / 32, TN = GATED ? 2 * TNO : TNO;
    constexpr int ROWS = BM + BN;           // 64-byte LDS rows per stage
    constexpr int STAGE_ELEMS = ROWS * BK;  // bf16 elements per stage
    constexpr int STAGE_BYTES = STAGE_ELEMS * 2;
    constexpr int NQ = ROWS / 64;  // 1 KB DMA instructions per wave per stage
    static_assert(TM >= 1 && TNO >= 1 && BM % 64 == 0 && BN % (GATED ? 128 : 64) == 0 && NS >= 4 && NS <= 9,
                  "tile shape");
    // one phase = max(MFMAs, fragment reads) pinned steps; a wave's DMAs go out every SP steps
    constexpr int STEPS_A = TM * TN > TM + TN ? TM * TN : TM + TN;
    constexpr int STEPS_B = STEPS_A;
    constexpr int SP = STEPS_A / (NQ - NQ / 2) > 0 ? STEPS_A / (NQ - NQ / 2) : 1;
    constexpr int SP0 = SP > 1 ? 1 : 0;
    static_assert(SP * (NQ - NQ / 2) <= STEPS_A, "DMA slots");

    // The tile-schedule scratch (1029 ints) lives at the start of the LDS ring: it is dead once the
    // tile is decoded, and the barrier below orders its last read before the first DMA write.
    static_assert(NS * STAGE_BYTES >= 1029 * 4 && NS * STAGE_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE_ELEMS];
    int* s_ts = reinterpret_cast<int*>(lds);
    int* s_wave = s_ts + 1025;

    if (offsets) build_schedule<BM, 256>(offsets, e_begin, n_groups, s_ts, s_wave);
    const TileCoord tc = decode_tile<BM, BNO, GM>(offsets, s_ts, e_begin, n_groups, dense_rows, n_out);
    if (!tc.valid) return;  // uniform per block
    __syncthreads();

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int64_t n_b_rows = GATED ? 2 * (int64_t)n_out : n_out;
    const uint16_t* Bg = B + (int64_t)tc.e * n_b_rows * K;
    const int64_t a_rows = tc.row_end - tc.row0 < BM ? tc.row_end - tc.row0 : BM;
    const int bn_part = GATED ? BN / 2 : BN;
    const int bcols = n_out - tc.n0 < bn_part ? n_out - tc.n0 : bn_part;
    // gathered rows: A holds the tokens and row p of the group is A[gather[p]]; the descriptor covers
    // all of A and each lane addresses its own row
    const i32x4 ra = gather ? make_rsrc(A, a_bytes) : make_rsrc(A + tc.row0 * K, (uint32_t)(a_rows * K * 2));
    const i32x4 rb0 = make_rsrc(Bg + (int64_t)tc.n0 * K, (uint32_t)((int64_t)bcols * K * 2));
    const i32x4 rb1 = make_rsrc(Bg + (int64_t)(GATED ? n_out + tc.n0 : tc.n0) * K, (uint32_t)((int64_t)bcols * K * 2));
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)lds;

    // DMA q of this wave covers LDS rows [(q * 4 + wave) * 16, +16) of a stage; lane -> (row, chunk)
    int voff[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int R = (q * 4 + wave) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swz(R);
        int row;
        if (q < BM / 64) row = R;
        else if (!GATED || q < (BM + BN / 2) / 64) row = R - BM;
        else row = R - BM - BN / 2;
        voff[q] = row * K * 2 + c * 16;
        if (q < BM / 64 && gather) voff[q] = gathered_voff(gather, tc.row0, tc.row_end, R, K, c);
    }
    // K not a multiple of BK (KT): the last stage's weight chunks past K read as zeros (the lane's
    // offset is pushed past the descriptor's range), so the token rows' bytes past K, which belong to
    // the next row, are multiplied by zero
    const int nk = KT ? (K + BK - 1) / BK : K / BK;
    int tor[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int R = (q * 4 + wave) * 16 + (lane >> 2);
        tor[q] = KT && q >= BM / 64 && ((lane & 3) ^ swz(R)) * 8 >= K - (nk - 1) * BK ? (int)0x80000000 : 0;
    }
    // operand rows of this lane
    int a_off[TM], a_sw[TM], b_off[TN], b_sw[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + i * 32 + (lane & 31);
        a_off[i] = r * BK;
        a_sw[i] = swz(r);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int jj = j < TNO ? j : j - TNO;
        const int r = BM + (GATED && j >= TNO ? BN / 2 : 0) + wn * WTNO + jj * 32 + (lane & 31);
        b_off[j] = r * BK;
        b_sw[j] = swz(r);
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

#define MOE_RSRC(q) ((q) < BM / 64 ? ra : ((!GATED || (q) < (BM + BN / 2) / 64) ? rb0 : rb1))
#define MOE_VOFF(q, kd_) (KT && (kd_) == nk - 1 ? (voff[q] | tor[q]) : voff[q])
#define MOE_ISSUE(kt_, q0, q1)                                                                            \
    {                                                                                                     \
        const int kt__ = (kt_);                                                                           \
        const uint32_t sbase = lds_base + (kt__ % NS) * STAGE_BYTES + wave * 1024;                        \
        const int soff = __builtin_amdgcn_readfirstlane(kt__ * BK * 2);                                   \
        _Pragma("unroll") for (int q = 0; q < NQ; ++q) if (q >= (q0) && q < (q1))                          \
            dma16(sbase + q * 4096, MOE_VOFF(q, kt__), MOE_RSRC(q), soff);                                \
    }
#define MOE_FREAD(slot_, kk, f)                                                                           \
    {                                                                                                     \
        const uint16_t* L_ = lds + (slot_) * STAGE_ELEMS;                                                 \
        const int c_ = (kk) * 2 + khalf;                                                                  \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) fa[f][i] =                                          \
            *reinterpret_cast<const bf16x8*>(L_ + a_off[i] + ((c_ ^ a_sw[i]) << 3));                      \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[f][j] =                                          \
            *reinterpret_cast<const bf16x8*>(L_ + b_off[j] + ((c_ ^ b_sw[j]) << 3));                      \
    }
#define MOE_MMA(f)                                                                                        \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) _Pragma("unroll") for (int j = 0; j < TN; ++j)         \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][i], fb[f][j], acc[i][j], 0, 0, 0);

    // DMA schedule: a stage's first NH instructions go out in phase B of one iteration and the rest in
    // phase A of the next, one every two MFMAs, so no wave bursts the vector-memory queue.
    constexpr int NH = NQ / 2;
    const bool split = nk >= NS;
    if (split) {
#pragma unroll
        for (int p = 0; p < NS - 2; ++p) MOE_ISSUE(p, 0, NQ);
        MOE_ISSUE(NS - 2, 0, NH);
        wait_vm<(NS - 3) * NQ + NH>();
    } else {
        for (int p = 0; p < nk; ++p) MOE_ISSUE(p, 0, NQ);
        wait_stages<NQ>(nk - 1);
    }
    lds_barrier();
    MOE_FREAD(0, 0, 0);
    int kt = 0;
    for (; kt + NS - 1 < nk; ++kt) {
        // phase A: MFMAs on the first K half of stage kt, reads of its second half, rest of stage kt+NS-2
        {
            const uint16_t* L1 = lds + (kt % NS) * STAGE_ELEMS;
            const int c1 = 2 + khalf;
            const int kd = kt + NS - 2;
            const uint32_t sbase = lds_base + (kd % NS) * STAGE_BYTES + wave * 1024;
            const int soff = __builtin_amdgcn_readfirstlane(kd * BK * 2);
#pragma unroll
            for (int t = 0; t < STEPS_A; ++t) {
                if (t < TM * TN)
                    acc[t / TN][t % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][t / TN], fb[0][t % TN],
                                                                                  acc[t / TN][t % TN], 0, 0, 0);
                if (t < TM) {
                    fa[1][t] = *reinterpret_cast<const bf16x8*>(L1 + a_off[t] + ((c1 ^ a_sw[t]) << 3));
                } else if (t < TM + TN) {
                    fb[1][t - TM] =
                        *reinterpret_cast<const bf16x8*>(L1 + b_off[t - TM] + ((c1 ^ b_sw[t - TM]) << 3));
                }
                if (t % SP == SP0 && NH + t / SP < NQ) {
                    const int q = NH + t / SP;
                    dma16(sbase + q * 4096, MOE_VOFF(q, kd), MOE_RSRC(q), soff);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // stage kt+1 has landed for every wave, and stage kt-1's slot is free for stage kt+NS-1
        wait_vm<(NS - 3) * NQ>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // phase B: MFMAs on the second half; reads of stage kt+1's first half; first half of stage kt+NS-1
        {
            const int kd = kt + NS - 1;
            const uint32_t sbase = lds_base + (kd % NS) * STAGE_BYTES + wave * 1024;
            const int soff = __builtin_amdgcn_readfirstlane(kd * BK * 2);
            const uint16_t* L0 = lds + ((kt + 1) % NS) * STAGE_ELEMS;
            const int c0 = khalf;
#pragma unroll
            for (int t = 0; t < STEPS_B; ++t) {
                if (t < TM * TN)
                    acc[t / TN][t % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][t / TN], fb[1][t % TN],
                                                                                  acc[t / TN][t % TN], 0, 0, 0);
                if (t < TM) {
                    fa[0][t] = *reinterpret_cast<const bf16x8*>(L0 + a_off[t] + ((c0 ^ a_sw[t]) << 3));
                } else if (t < TM + TN) {
                    fb[0][t - TM] =
                        *reinterpret_cast<const bf16x8*>(L0 + b_off[t - TM] + ((c0 ^ b_sw[t - TM]) << 3));
                }
                if (t % SP == SP0 && t / SP < NH) {
                    const int q = t / SP;
                    dma16(sbase + q * 4096, MOE_VOFF(q, kd), MOE_RSRC(q), soff);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (split) MOE_ISSUE(nk - 1, NH, NQ);  // rest of the last stage
    for (; kt < nk; ++kt) {  // the last NS - 1 stages (all issued)
        MOE_FREAD(kt % NS, 1, 1);
        MOE_MMA(0);
        if (kt + 1 < nk) wait_stages<NQ>(nk - kt - 2);
        lds_barrier();
        if (kt + 1 < nk) MOE_FREAD((kt + 1) % NS, 0, 0);
        MOE_MMA(1);
    }
#undef MOE_ISSUE
#undef MOE_VOFF
#undef MOE_RSRC
#undef MOE_FREAD
#undef MOE_MMA

    // Epilogue. 32x32 accumulator: lane holds column lane%32 and rows 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TNO; ++j) {
            const int col = tc.n0 + wn * WTNO + j * 32 + (lane & 31);
            if (col >= n_out) continue;
            float bcol = 0.f;
            if (EPI != EPI_SWIGLU && bias != nullptr) bcol = bf16_to_f32(bias[(int64_t)tc.e * n_out + col]);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = tc.row0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
                if (row >= tc.row_end) continue;
                if (EPI == EPI_F32) {  // fp32 output (dense products only)
                    reinterpret_cast<float*>(C)[row * n_out + col] = acc[i][j][v];
                    continue;
                }
                float out;
                if (EPI == EPI_SWIGLU) out = silu_f(acc[i][j][v]) * acc[i][j + TNO][v];
                else if (EPI == EPI_GELU_BIAS) out = gelu_f(acc[i][j][v] + bcol);
                else out = acc[i][j][v] + bcol;
                C[row * n_out + col] = f32_to_bf16(out);
            }
        }
    }
}

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cu_count() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Tile schedule of the persistent GEMM and its tail fixup: the expert-major tile order, each
// XCD's contiguous chunk of it, and how that chunk is dealt to the XCD's blocks.
template <int BM, int BNO, int GM>
struct TileSched {
    const int* s_ts;   // LDS: row-tile prefix sums per group (grouped)
    const int* s_off;  // LDS: offsets[e_begin .. e_begin + n_groups] (grouped)
    bool grouped;
    int e_begin, n_groups;
    int64_t dense_rows;
    uint32_t n_tiles_n, m_tiles, R;

    // lin -> tile; inside an expert, groups of GM row tiles sweep the column tiles (row tile fastest)
    __device__ __forceinline__ void decode(uint32_t lin, int64_t& row0, int64_t& row_end, int& e, int& n0) const {
        int g = 0;
        uint32_t g_mt = m_tiles, local = lin;
        if (grouped) {
            const uint32_t key = lin / n_tiles_n;
            int lo = 0, hi = n_groups - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((uint32_t)s_ts[mid] <= key) lo = mid;
                else hi = mid - 1;
            }
            g = lo;
            g_mt = (uint32_t)(s_ts[g + 1] - s_ts[g]);
            local = lin - (uint32_t)s_ts[g] * n_tiles_n;
        }
        const uint32_t grp_ = local / (GM * n_tiles_n);
        const uint32_t first_m = grp_ * GM;
        const uint32_t gsz = g_mt - first_m < GM ? g_mt - first_m : GM;
        const uint32_t rem = local - grp_ * GM * n_tiles_n;
        const uint32_t col = rem / gsz;
        const uint32_t mt = first_m + (rem - col * gsz);
        n0 = (int)col * BNO;
        if (grouped) {
            e = e_begin + g;
            row0 = s_off[g] + (int64_t)mt * BM;
            row_end = s_off[g + 1];
        } else {
            e = 0;
            row0 = (int64_t)mt * BM;
            row_end = dense_rows;
        }
    }
};

// Split of one XCD's chunk over its nslots blocks: every block takes nwhole whole tiles; the rem
// tiles left over are cut along K into S slices each (S >= 2, rem * S <= nslots) when a partial
// buffer is given, so the last round keeps every CU busy; otherwise the first rem blocks take one
// more whole tile.
struct XcdPlan {
    uint32_t chunk0, nwhole, rem, S;
};
__device__ __forceinline__ XcdPlan xcd_plan(uint32_t R, uint32_t xcd, uint32_t nslots, int nk, bool split) {
    const uint32_t per = (R + 7) / 8;
    const uint32_t c0 = xcd * per;
    const uint32_t c1 = (xcd + 1) * per < R ? (xcd + 1) * per : R;
    const uint32_t C = c1 > c0 ? c1 - c0 : 0;
    XcdPlan p;
    p.chunk0 = c0;
    p.nwhole = C / nslots;
    p.rem = C - p.nwhole * nslots;
    p.S = 1;
    if (split && p.rem > 0) {
        uint32_t S = nslots / p.rem;
        if (S > (uint32_t)nk) S = (uint32_t)nk;
        p.S = S >= 2 ? S : 1;
    }
    return p;
}

// Build the schedule in LDS (a block of NT threads) and fill a TileSched.
template <int BM, int BNO, int GM, int NT = 512>
__device__ __forceinline__ TileSched<BM, BNO, GM> setup_sched(const int32_t* __restrict__ offsets, int e_begin,
                                                              int n_groups, int64_t dense_rows, int n_out,
                                                              int* s_ts, int* s_off, int* s_wave) {
    if (offsets) {
        for (int g = threadIdx.x; g <= n_groups; g += NT) s_off[g] = offsets[e_begin + g];
        build_schedule<BM, NT>(offsets, e_begin, n_groups, s_ts, s_wave);  // ends with a barrier
    }
    TileSched<BM, BNO, GM> ts;
    ts.s_ts = s_ts;
    ts.s_off = s_off;
    ts.grouped = offsets != nullptr;
    ts.e_begin = e_begin;
    ts.n_groups = n_groups;
    ts.dense_rows = dense_rows;
    // Tile counts fit 32 bits: rows <= T * k <= 2^31 - 1 and at most 2^31 / 128 column tiles.
    ts.n_tiles_n = (uint32_t)((n_out + BNO - 1) / BNO);
    ts.m_tiles = offsets ? (uint32_t)s_ts[n_groups] : (uint32_t)((dense_rows + BM - 1) / BM);
    ts.R = ts.m_tiles * ts.n_tiles_n;
    return ts;
}

// The same schedule held in registers instead of LDS, for kernels whose LDS ring takes all of it: at
// most kRegSchedGroups groups; entry g < n_groups of s_ts and of offsets[e_begin ..] sits in lane
// g % 64 of register g / 64 of every wave, entry n_groups (the totals) in scalars. Each wave forms it
// on its own (a wave-wide scan), and decode finds the group with ballots, so it must be called by
// whole waves.
constexpr int kRegSchedGroups = 128;
template <int BM, int BNO, int GM>
struct TileSchedR {
    int ts_l[2], off_l[2];
    int off_end;  // offsets[e_begin + n_groups]
    bool grouped;
    int e_begin, n_groups;
    int64_t dense_rows;
    uint32_t n_tiles_n, m_tiles, R;

    // entry g (uniform, g <= n_groups); entry n_groups is `last`
    __device__ __forceinline__ int at(const int (&v)[2], int g, int last) const {
        if (g >= n_groups) return last;
        return g < kWave ? __builtin_amdgcn_readlane(v[0], g) : __builtin_amdgcn_readlane(v[1], g - kWave);
    }
    __device__ __forceinline__ void decode(uint32_t lin, int64_t& row0, int64_t& row_end, int& e, int& n0) const {
        int g = 0;
        uint32_t g_mt = m_tiles, local = lin;
        if (grouped) {
            const uint32_t key = lin / n_tiles_n;
            // s_ts is non-decreasing: the last group whose first row tile is at or before key
            const int lane = lane_id();
            const uint64_t m0 = __ballot(lane < n_groups && (uint32_t)ts_l[0] <= key);
            const uint64_t m1 = __ballot(lane + kWave < n_groups && (uint32_t)ts_l[1] <= key);
            g = __builtin_amdgcn_readfirstlane(__popcll(m0) + __popcll(m1) - 1);
            const uint32_t t0 = (uint32_t)at(ts_l, g, (int)m_tiles);
            g_mt = (uint32_t)at(ts_l, g + 1, (int)m_tiles) - t0;
            local = lin - t0 * n_tiles_n;
        }
        const uint32_t grp_ = local / (GM * n_tiles_n);
        const uint32_t first_m = grp_ * GM;
        const uint32_t gsz = g_mt - first_m < GM ? g_mt - first_m : GM;
        const uint32_t rem = local - grp_ * GM * n_tiles_n;
        const uint32_t col = rem / gsz;
        const uint32_t mt = first_m + (rem - col * gsz);
        n0 = (int)col * BNO;
        if (grouped) {
            e = e_begin + g;
            row0 = at(off_l, g, off_end) + (int64_t)mt * BM;
            row_end = at(off_l, g + 1, off_end);
        } else {
            e = 0;
            row0 = (int64_t)mt * BM;
            row_end = dense_rows;
        }
    }
};
template <int BM, int BNO, int GM>
__device__ __forceinline__ TileSchedR<BM, BNO, GM> setup_sched_regs(const int32_t* __restrict__ offsets,
                                                                    int e_begin, int n_groups, int64_t dense_rows,
                                                                    int n_out) {
    TileSchedR<BM, BNO, GM> ts;
    const int lane = lane_id();
    ts.m_tiles = (uint32_t)((dense_rows + BM - 1) / BM);
    ts.n_groups = n_groups;
    ts.off_end = 0;
    int carry = 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        ts.ts_l[r] = 0;
        ts.off_l[r] = 0;
        if (!offsets) continue;
        const int g = r * kWave + lane;
        const int o = g < n_groups ? offsets[e_begin + g] : 0;
        const int o1 = g < n_groups ? offsets[e_begin + g + 1] : o;
        const int n = (o1 - o + BM - 1) / BM;
        int inc = n;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_up(inc, d, kWave);
            if (lane >= d) inc += v;
        }
        ts.ts_l[r] = carry + inc - n;  // exclusive prefix
        ts.off_l[r] = o;
        carry += __builtin_amdgcn_readlane(inc, kWave - 1);
    }
    if (offsets) {
        ts.m_tiles = (uint32_t)carry;
        ts.off_end = offsets[e_begin + n_groups];
    }
    ts.grouped = offsets != nullptr;
    ts.e_begin = e_begin;
    ts.dense_rows = dense_rows;
    ts.n_tiles_n = (uint32_t)((n_out + BNO - 1) / BNO);
    ts.R = ts.m_tiles * ts.n_tiles_n;
    return ts;
}

// Epilogue of one 32-token row block of a wave: a[j] holds a (feature x token) 32 x 32 block; a lane
// owns token `row` and, per group of 4 registers, 4 consecutive features from fbase + j * 32. FENCE
// keeps each group's reads of the accumulators next to its stores (for accumulators held in the
// AGPR file, so the copies out of it do not pile up in VGPRs).
// One accumulator value copied out of the AGPR file: the operand constraint keeps the accumulators
// in AGPRs where the epilogue's arithmetic would otherwise pull them into VGPRs.
__device__ __forceinline__ float from_agpr(float x) {
    float y;
    asm("v_accvgpr_read_b32 %0, %1" : "=v"(y) : "a"(x));
    return y;
}
// The same for accumulators held in VGPRs (where the AGPR file cannot hold them all).
__device__ __forceinline__ float from_vgpr(float x) {
    float y;
    asm("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}
// Accumulator j of a row block: the first NAG in AGPRs, the rest in VGPRs.
template <int NAG>
__device__ __forceinline__ float acc_read(int j, float x) {
    return j < NAG ? from_agpr(x) : from_vgpr(x);
}
// Global-memory views of the epilogue's destinations. The stores must be global, not flat: a flat
// store also counts on the LDS counter, so a later wait for fragment reads would wait for the stores
// as well. (A pointer passed through an empty asm loses its address space: the wide kernel's K-split
// partial stores compiled to flat stores before this cast.)
typedef __attribute__((address_space(1))) floatx4 global_floatx4;
__device__ __forceinline__ global_floatx4* as_global(floatx4* p) { return (global_floatx4*)p; }
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}
template <int EPI, int TN, bool FENCE = false, int NAG = TN>
__device__ __forceinline__ void store_block(const floatx16 (&a)[TN], int64_t row, int64_t row_end, int e,
                                            int fbase, int lane, uint16_t* __restrict__ C,
                                            const uint16_t* __restrict__ bias, int n_out) {
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int TNO = GATED ? TN / 2 : TN;
    const int khalf = lane >> 5;
    auto rd = [&](int jj, float x) { return FENCE ? acc_read<NAG>(jj, x) : x; };
    auto group = [&](int j, int q4, float (&o)[4]) {
        const int f0 = fbase + j * 32 + 8 * q4 + 4 * khalf;
        if (GATED) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float z = rd(j, a[j][4 * q4 + c]);
                o[c] = z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) * rd(j + TNO, a[j + TNO][4 * q4 + c]);
            }
        } else {
            float bc[4] = {0.f, 0.f, 0.f, 0.f};
            if (bias != nullptr && f0 < n_out) {
                const uint2 bb = *reinterpret_cast<const uint2*>(bias + (int64_t)e * n_out + f0);
                bc[0] = __uint_as_float(bb.x << 16);
                bc[1] = __uint_as_float(bb.x & 0xffff0000u);
                bc[2] = __uint_as_float(bb.y << 16);
                bc[3] = __uint_as_float(bb.y & 0xffff0000u);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float z = rd(j, a[j][4 * q4 + c]) + bc[c];
                o[c] = EPI == EPI_GELU_BIAS ? gelu_f(z) : z;
            }
        }
    };
#pragma unroll
    for (int j = 0; j < TNO; ++j) {
        if (EPI == EPI_F32) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int f0 = fbase + j * 32 + 8 * q4 + 4 * khalf;
                if (row < row_end && f0 < n_out)
                    *as_global(reinterpret_cast<floatx4*>(reinterpret_cast<float*>(C) + row * n_out + f0)) =
                        floatx4{rd(j, a[j][4 * q4]), rd(j, a[j][4 * q4 + 1]), rd(j, a[j][4 * q4 + 2]),
                                rd(j, a[j][4 * q4 + 3])};
            }
            continue;
        }
        // groups q4 = 2 qp and 2 qp + 1: a lane holds features 16 qp + 8 q + 4 khalf + [0, 4) of each; one
        // swap between the wave's halves leaves lane l < 32 with features 16 qp + [0, 8) and lane l + 32
        // with 16 qp + [8, 16) of the same token, so each lane writes 16 contiguous bytes
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
            float oP[4], oQ[4];
            group(j, 2 * qp, oP);
            group(j, 2 * qp + 1, oQ);
            const auto s0 = __builtin_amdgcn_permlane32_swap(pack2_bf16(oP[0], oP[1]), pack2_bf16(oQ[0], oQ[1]),
                                                             false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(pack2_bf16(oP[2], oP[3]), pack2_bf16(oQ[2], oQ[3]),
                                                             false, false);
            const int f = fbase + j * 32 + 16 * qp + 8 * khalf;
            if (row < row_end && f < n_out) {
                uint4 pk;
                pk.x = s0[0];
                pk.y = s1[0];
                pk.z = s0[1];
                pk.w = s1[1];
                *reinterpret_cast<uint4*>(C + row * n_out + f) = pk;
            }
            if (FENCE) __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Eight-wave tile layouts. A wave (group grp, wm, wn) owns 64 tokens x TNO * 32 features (and, for
// SwiGLU, the matching up features). 256-row tiles: the groups take tokens [0, 128) and [128, 256)
// of the same features. 128-row tiles (R128): both groups take all 128 tokens, each its own half of
// the tile's features.
template <bool R128>
__device__ __forceinline__ int wave_row_base(int grp, int wm) { return (R128 ? 0 : grp * 128) + wm * 64; }
template <bool R128, int WTNO>
__device__ __forceinline__ int wave_feat_base(int grp, int wn) { return (R128 ? grp * 2 * WTNO : 0) + wn * WTNO; }

// Epilogue of one wave's block of a tile (eight-wave layouts): acc[i] is the row block of tokens
// wave_row_base + i * 32, features from n0 + wave_feat_base.
template <int EPI, int TM, int TN, bool R128>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[TM][TN], int64_t row0, int64_t row_end, int e,
                                           int n0, int grp, int wm, int wn, int lane,
                                           uint16_t* __restrict__ C, const uint16_t* __restrict__ bias,
                                           int n_out) {
    constexpr int TNO = EPI == EPI_SWIGLU ? TN / 2 : TN, WTNO = TNO * 32;
#pragma unroll
    for (int i = 0; i < TM; ++i)
        store_block<EPI, TN>(acc[i], row0 + wave_row_base<R128>(grp, wm) + i * 32 + (lane & 31), row_end, e,
                             n0 + wave_feat_base<R128, WTNO>(grp, wn), lane, C, bias, n_out);
}

// Partial buffer: a header, then the fp32 accumulators of each tile slice as
// [slot][wave][i][j][v / 4][lane] float4 (each store and load moves 1 KB per wave instruction).
// Header: per XCD {rem, S} of its split last round, and per tail tile {row0, row_end, e, n0}.
constexpr int kPartialFloats = 256 * (kGemmWideBN > 256 ? kGemmWideBN : 256);  // one output tile
constexpr int kMaxSlotsPerXcd = 64;        // nslots <= 64 (512 blocks)
struct TailTile {
    int64_t row0, row_end;
    int32_t e, n0;
};
struct TailHeader {
    int32_t rem[8], S[8];
    TailTile tile[8][kMaxSlotsPerXcd];
};
constexpr size_t kTailHeaderBytes = (sizeof(TailHeader) + 255) / 256 * 256;
template <int TM, int TN>
__device__ __forceinline__ floatx4* partial_at(float* partials, uint32_t pslot, int wave) {
    float* slots = partials + kTailHeaderBytes / sizeof(float);
    return reinterpret_cast<floatx4*>(slots + (size_t)pslot * kPartialFloats) + (size_t)wave * (TM * TN * 4 * 64);
}

// Persistent form of the eight-wave ping-pong tile: one block per CU walks its share of the tile
// sequence, so the tile schedule and the expert offsets are read into LDS once per block, and the
// LDS ring runs on across tile boundaries (the next tile's first stages arrive while the current
// tile's last stages are multiplied). Blocks are dealt to XCDs round-robin; the 32 blocks of an XCD
// take 32 consecutive tiles of that XCD's chunk at a time (GM row tiles x 32/GM column tiles of one
// expert), so they share weight panels and token tiles through the XCD's L2 while running in step.
// When the chunk does not divide into whole rounds, the tiles of the last round are cut along K
// and spread over all the XCD's blocks (see xcd_plan); those slices leave fp32 partial tiles that
// gemm_bf16_tail_kernel sums in slice order, so the result does not depend on timing.
//
// The MFMA operands are the weight fragment first and the token fragment second, so an accumulator
// holds a (feature x token) block: a lane owns one token and, per group of 4 registers, 4
// consecutive output features, written with one 8-byte store. Stores and LDS-DMA loads share the
// vector-memory counter and may complete out of order, so the memory cluster after a tile's stores
// waits for the counter to drain before it issues new loads.
//
// R128: 128-token x 512-weight-row tiles for small expert groups (a few hundred rows or less, where
// 256-row tiles are mostly padding): both groups multiply the same 128 tokens, each against its own
// 256 weight rows, so a wave's block and the MFMA work per stage are those of the 256-row tile. A
// stage is then 640 rows (40 KB), five DMA instructions per wave, and the ring holds D + 1 = 3
// stages.
template <int EPI, int GM, int D, bool KT, bool R128, bool GA>
__global__ __launch_bounds__(512, 1) void gemm_bf16_persistent_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ C, const int32_t* __restrict__ offsets, int e_begin, int n_groups, int64_t dense_rows,
    int n_out, int K, float* __restrict__ partials, const int32_t* __restrict__ gather, uint32_t a_bytes) {
    constexpr int BM = R128 ? 128 : 256, BN = R128 ? 512 : 256, BK = 32, NS = D + 1;
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int TM = 2;  // 64 tokens per wave
    constexpr int BNO = GATED ? BN / 2 : BN, WTNO = R128 ? BNO / 4 : BNO / 2, TNO = WTNO / 32;
    constexpr int TN = GATED ? 2 * TNO : TNO;
    constexpr int STAGE_ELEMS = (BM + BN) * BK;  // 512 (R128: 640) rows of 64 bytes
    constexpr int STAGE_BYTES = STAGE_ELEMS * 2;
    // DMA instructions per wave per stage, 16 rows each. 256-row tiles: group 0 moves the 256 token
    // rows, group 1 the 256 weight rows. R128: instruction q of wave w moves stage rows
    // (q * 8 + w) * 16 + [0, 16), so q = 0 covers the 128 token rows and q >= 1 the weight rows.
    constexpr int NQ = R128 ? 5 : 4;
    static_assert(TN == 4 && D >= 2 && D <= 5, "tile shape");
    static_assert(NS * STAGE_BYTES + 2 * 1025 * 4 + 8 * 4 <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE_ELEMS];
    __shared__ int s_ts[1025];
    __shared__ int s_off[1025];
    __shared__ int s_wave[8];

    const int tid = threadIdx.x, lane = lane_id();
    const TileSched<BM, BNO, GM> ts =
        setup_sched<BM, BNO, GM>(offsets, e_begin, n_groups, dense_rows, n_out, s_ts, s_off, s_wave);
    const int nk = KT ? (K + BK - 1) / BK : K / BK;
    const uint32_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
    const XcdPlan plan = xcd_plan(ts.R, xcd, nslots, nk, partials != nullptr);
    // this block's units: nw whole tiles, then at most one K slice of a tail tile
    const uint32_t nw = plan.nwhole + ((plan.S == 1 && slot < plan.rem) ? 1u : 0u);
    const bool has_slice = plan.S >= 2 && slot < plan.rem * plan.S;
    const uint32_t slice_lin = plan.chunk0 + plan.nwhole * nslots + (has_slice ? slot / plan.S : 0);
    const int slice_part = has_slice ? (int)(slot % plan.S) : 0;
    const int slice_kb = slice_part * nk / (int)plan.S, slice_ke = (slice_part + 1) * nk / (int)plan.S;
    const int nunits = (int)nw + (has_slice ? 1 : 0);
    if (partials != nullptr && tid == 0) {
        TailHeader* hdr = reinterpret_cast<TailHeader*>(partials);
        if (slot == 0) {
            hdr->rem[xcd] = (int32_t)plan.rem;
            hdr->S[xcd] = (int32_t)plan.S;
        }
        if (has_slice && slice_part == 0) {
            TailTile tt;
            ts.decode(slice_lin, tt.row0, tt.row_end, tt.e, tt.n0);
            hdr->tile[xcd][slot / plan.S] = tt;
        }
    }
    if (nunits == 0) return;  // uniform per block
    auto unit_lin = [&](int u) { return u < (int)nw ? plan.chunk0 + slot + (uint32_t)u * nslots : slice_lin; };
    auto unit_kb = [&](int u) { return u < (int)nw ? 0 : slice_kb; };
    auto unit_ke = [&](int u) { return u < (int)nw ? nk : slice_ke; };

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wig = wave & 3;
    const int wm = wig & 1, wn = wig >> 1;
    const int64_t n_b_rows = GATED ? 2 * (int64_t)n_out : n_out;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)lds;

    // DMA q of this wave: 16 stage rows (see NQ); lane -> (row, chunk). Row offsets are relative to
    // the tile's buffer descriptors, so they hold for every tile.
    // stage row of DMA q, this lane; whether it is a weight row; its row in its descriptor
    auto dma_row0 = [&](int q) { return R128 ? (q * 8 + wave) * 16 : grp * 256 + (q * 4 + wig) * 16; };  // uniform
    auto dma_row = [&](int q) { return dma_row0(q) + (lane >> 2); };
    auto dma_is_b = [&](int q) { return R128 ? q >= 1 : grp == 1; };
    auto dma_desc_row = [&](int q) {
        const int R = dma_row(q);
        if (!dma_is_b(q)) return R;
        const int b = R - BM;  // weight row of the tile: gate rows, then (SwiGLU) the matching up rows
        return GATED && b >= BNO ? b - BNO : b;
    };
    int voff[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) voff[q] = dma_desc_row(q) * K * 2 + ((lane & 3) ^ swz(dma_row(q))) * 16;
    // K not a multiple of BK (KT): the weight chunks of the last stage past K read as zeros
    int tor[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        tor[q] = KT && dma_is_b(q) && ((lane & 3) ^ swz(dma_row(q))) * 8 >= K - (nk - 1) * BK ? (int)0x80000000 : 0;
    // buffer descriptors of the tile whose stages are being loaded
    i32x4 rs[NQ];
    auto set_dma_tile = [&](uint32_t lin) {
        int64_t row0, row_end;
        int e, n0;
        ts.decode(lin, row0, row_end, e, n0);
        if (R128 || grp == 0) {
            const int64_t a_rows = row_end - row0 < BM ? row_end - row0 : BM;
            const i32x4 ra = GA ? make_rsrc(A, a_bytes) : make_rsrc(A + row0 * K, (uint32_t)(a_rows * K * 2));
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (!dma_is_b(q)) {
                    rs[q] = ra;
                    if (GA)  // gathered token rows: this tile's row offsets
                        voff[q] = gathered_voff_uniform<16>(gather, row0, row_end, dma_row0(q), K);
                }
        }
        if (R128 || grp == 1) {
            const uint16_t* Bg = B + (int64_t)e * n_b_rows * K;
            const int bcols = n_out - n0 < BNO ? n_out - n0 : BNO;
            const i32x4 rb0 = make_rsrc(Bg + (int64_t)n0 * K, (uint32_t)((int64_t)bcols * K * 2));
            const i32x4 rb1 =
                make_rsrc(Bg + (int64_t)(GATED ? n_out + n0 : n0) * K, (uint32_t)((int64_t)bcols * K * 2));
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (dma_is_b(q)) rs[q] = (GATED && dma_row0(q) - BM >= BNO) ? rb1 : rb0;
        }
    };

    int a_off[TM], a_sw[TM], b_off[TN], b_sw[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wave_row_base<R128>(grp, wm) + i * 32 + (lane & 31);
        a_off[i] = r * BK;
        a_sw[i] = swz(r);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int jj = j < TNO ? j : j - TNO;
        const int r = BM + (GATED && j >= TNO ? BNO : 0) + wave_feat_base<R128, WTNO>(grp, wn) + jj * 32 + (lane & 31);
        b_off[j] = r * BK;
        b_sw[j] = swz(r);
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

    // stage counters are kept incrementally (no division in the loop): slot in the ring, K slice
    // in the unit
#define PS_ISSUE(slot_, ks_)                                                                              \
    {                                                                                                     \
        const uint32_t sbase = lds_base + (slot_) * STAGE_BYTES + (R128 ? wave : grp * 16 + wig) * 1024;  \
        const int soff = (ks_) * (BK * 2);                                                                \
        const bool tail_ = KT && (ks_) == nk - 1;                                                         \
        _Pragma("unroll") for (int q = 0; q < NQ; ++q)                                                    \
            dma16(sbase + q * (R128 ? 8192 : 4096), tail_ ? (voff[q] | tor[q]) : voff[q], rs[q], soff);   \
    }
#define PS_READ(slot_)                                                                                    \
    {                                                                                                     \
        const uint16_t* L_ = lds + (slot_) * STAGE_ELEMS;                                                 \
        _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                                \
            const int c_ = kk * 2 + khalf;                                                                \
            _Pragma("unroll") for (int i = 0; i < TM; ++i) fa[kk][i] =                                     \
                *reinterpret_cast<const bf16x8*>(L_ + a_off[i] + ((c_ ^ a_sw[i]) << 3));                  \
            _Pragma("unroll") for (int j = 0; j < TN; ++j) fb[kk][j] =                                     \
                *reinterpret_cast<const bf16x8*>(L_ + b_off[j] + ((c_ ^ b_sw[j]) << 3));                  \
        }                                                                                                 \
    }
#define PS_MMA                                                                                            \
    _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) _Pragma("unroll") for (int i = 0; i < TM; ++i)       \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                    \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk][j], fa[kk][i], acc[i][j], 0, 0, 0);

    int G = (int)nw * nk + (has_slice ? slice_ke - slice_kb : 0);  // stages of all this block's units
    const int npro = G < D ? G : D;
    int dma_u = 0;  // unit whose stages are being issued
    set_dma_tile(unit_lin(0));
    int w_slot = 0, w_ks = unit_kb(0), w_ke = unit_ke(0);
    auto dma_advance = [&]() {
        w_slot = w_slot + 1 == NS ? 0 : w_slot + 1;
        if (++w_ks == w_ke && dma_u + 1 < nunits) {
            ++dma_u;
            set_dma_tile(unit_lin(dma_u));
            w_ks = unit_kb(dma_u);
            w_ke = unit_ke(dma_u);
        }
    };
    for (int p = 0; p < npro; ++p) {
        PS_ISSUE(w_slot, w_ks)
        dma_advance();
    }
    wait_stages<NQ>(npro - 1);  // stage 0 of this wave has landed
    lds_barrier();
    if (grp == 1) lds_barrier();  // group 1 runs one cluster behind group 0
    __builtin_amdgcn_sched_barrier(0);

    int cmp_u = 0;        // unit being multiplied
    bool drain = false;   // stores of the previous unit may be in flight
    int r_slot = 0, r_ks = unit_kb(0), r_ke = unit_ke(0);
    for (int g = 0; g < G; ++g) {
        // memory cluster: fragments of stage g, loads of stage g + D
        PS_READ(r_slot)
        if (drain) {
            wait_vm<0>();
            drain = false;
        }
        if (g + D < G) {
            PS_ISSUE(w_slot, w_ks)
            dma_advance();
            wait_vm<(D - 1) * NQ>();  // stage g + 1 of this wave has landed
        } else {
            wait_stages<NQ>(G - g - 2);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // compute cluster, at raised issue priority so the partner wave's memory cluster on the same
        // SIMD does not delay an MFMA issue (measured: down projection about 2 % faster)
        __builtin_amdgcn_s_setprio(1);
        PS_MMA
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        r_slot = r_slot + 1 == NS ? 0 : r_slot + 1;
        if (++r_ks == r_ke) {  // last stage of a unit: store it
            if (cmp_u < (int)nw) {
                int64_t row0, row_end;
                int e, n0;
                ts.decode(unit_lin(cmp_u), row0, row_end, e, n0);
                store_tile<EPI, TM, TN, R128>(acc, row0, row_end, e, n0, grp, wm, wn, lane, C, bias, n_out);
            } else {
                floatx4* dst = partial_at<TM, TN>(partials, xcd * nslots + slot, wave);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int v4 = 0; v4 < 4; ++v4)
                            dst[((i * TN + j) * 4 + v4) * 64 + lane] =
                                floatx4{acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2],
                                        acc[i][j][4 * v4 + 3]};
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
            drain = true;
            if (cmp_u + 1 < nunits) {
                ++cmp_u;
                r_ks = unit_kb(cmp_u);
                r_ke = unit_ke(cmp_u);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }
    if (grp == 0) lds_barrier();
#undef PS_ISSUE
#undef PS_READ
#undef PS_MMA
}

// K-grouped products (the weight gradients): one dense product per expert, C_e = A_e B_e^T, whose K
// range is the expert's column range [poff[e], poff[e + 1]) of A and B (both [rows][ld], K
// contiguous; each range a multiple of 64, zero-padded). The experts' output rows are stacked (row
// e * m_per_e + m of C), m_per_e a multiple of 256, so a tile never spans two experts.
struct KgArgs {
    const int32_t* poff;
    int64_t ld;
    int m_per_e;
};

// Four-wave, wide-K form of the persistent GEMM, for large groups: the tile sequence, XCD plan and K
// split of the eight-wave kernel, with each wave owning a 128-token x BN / 2-weight-row block of the
// tile (one wave per SIMD) and the memory instructions placed between the wave's own MFMAs instead of
// in a partner wave's cluster. Stages are 64 columns wide (128-byte LDS rows, a two-slot ring), so each
// DMA instruction reads 8 whole 128-byte row pieces instead of 16 half lines. Chunk c of LDS row r
// sits at position c ^ ((r / 2) % 8), which keeps the 16-lane groups of a fragment read on distinct
// banks. A stage is four 16-wide K steps; the DMAs of the next stage go out during the first two (one
// after every other MFMA), and the last step waits for them, passes the stage barrier and reads the
// next stage's first fragments. K-split slices store their partial tiles in the eight-wave layout
// (with BN / 64 column blocks per wave) that gemm_bf16_tail_kernel reads.
//
// BN = 384 weight rows: 24 accumulators of 32 x 32 per wave, 384 registers, more than the 256 of the
// AGPR file, so acc[i][4..5] live in VGPRs (fragments and addresses take the other 120 or so). A
// stage is 80 KB, the two slots take all 160 KB of LDS, and the tile schedule lives in registers
// (TileSchedR, at most 128 groups). Per MFMA, a stage moves 17 % fewer operand bytes than with
// BN = 256, and each stage is half as long again, which covers more of the next stage's DMA latency.

template <int EPI, int GM, bool KT, bool GA, int BN, bool KG>
__global__ __launch_bounds__(256, 1) void gemm_bf16_wide_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ C, const int32_t* __restrict__ offsets, int e_begin, int n_groups, int64_t dense_rows,
    int n_out, int K, float* __restrict__ partials, const int32_t* __restrict__ gather, uint32_t a_bytes,
    KgArgs kg) {
    constexpr int BM = 256, BK = 64, NS = 2;
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int TM = 4;
    constexpr int BNO = GATED ? BN / 2 : BN, WTNO = BNO / 2, TNO = WTNO / 32, TN = GATED ? 2 * TNO : TNO;
    constexpr int STAGE_ELEMS = (BM + BN) * BK;  // BM + BN rows of 128 bytes
    constexpr int STAGE_BYTES = STAGE_ELEMS * 2;
    constexpr int NQ = (BM + BN) / 32;  // DMA instructions per wave per stage (8 rows each)
    constexpr int QUP = BM / 32 + BN / 64;  // first DMA on the up rows (SwiGLU)
    constexpr int NF = TM + TN;             // fragment reads per 16-wide K step
    constexpr int NT = TM * TN;             // MFMAs per 16-wide K step
    // accumulators: 16 blocks of 32 x 32 fill the AGPR file; with 384 weight rows acc[i][4..5] are in VGPRs
    constexpr int NAG = 16 / TM;
    // MFMAs of the last K step before the wait for the next stage's DMAs: with 24 per step, the latest
    // point that leaves one MFMA per fragment read of the next stage's first step (measured on the
    // Mixtral-shaped layer against 6, 10 and 12: step 4.75, 4.71, 4.66 and 4.62 ms for 14)
    constexpr int WB = BN > 256 ? NT - NF : TN;
    // 384-row weight tiles fill the LDS with the ring; their tile schedule is held in registers
    constexpr bool RS = BN > 256;
    constexpr int SCHED_ELEMS = RS ? 0 : (2 * 1025 + 8) * 2;
    static_assert(TN == BN / 64 && BN % 128 == 0 && NF <= NT / 2 && NQ - NQ / 2 <= NT / 2 && NF <= NT - WB,
                  "tile shape");
    static_assert(NS * STAGE_BYTES + SCHED_ELEMS * 2 <= 160 * 1024, "LDS budget");
    static_assert(!KG || (EPI == EPI_F32 && !KT && !GA), "K-grouped products: fp32 output, K in whole stages");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE_ELEMS + SCHED_ELEMS];

    const int tid = threadIdx.x, lane = lane_id();
    using Sched = typename std::conditional<RS, TileSchedR<BM, BNO, GM>, TileSched<BM, BNO, GM>>::type;
    Sched ts;
    if constexpr (RS) {
        ts = setup_sched_regs<BM, BNO, GM>(offsets, e_begin, n_groups, dense_rows, n_out);
    } else {
        int* s_ts = reinterpret_cast<int*>(lds + NS * STAGE_ELEMS);
        ts = setup_sched<BM, BNO, GM, 256>(offsets, e_begin, n_groups, dense_rows, n_out, s_ts, s_ts + 1025,
                                           s_ts + 2050);
    }
    const int nk = KT ? (K + BK - 1) / BK : K / BK;
    const uint32_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
    const XcdPlan plan = xcd_plan(ts.R, xcd, nslots, nk, partials != nullptr);
    const uint32_t nw = plan.nwhole + ((plan.S == 1 && slot < plan.rem) ? 1u : 0u);
    const bool has_slice = plan.S >= 2 && slot < plan.rem * plan.S;
    const uint32_t slice_lin = plan.chunk0 + plan.nwhole * nslots + (has_slice ? slot / plan.S : 0);
    const int slice_part = has_slice ? (int)(slot % plan.S) : 0;
    const int slice_kb = slice_part * nk / (int)plan.S, slice_ke = (slice_part + 1) * nk / (int)plan.S;
    const int nunits = (int)nw + (has_slice ? 1 : 0);
    if (partials != nullptr) {
        TailHeader* hdr = reinterpret_cast<TailHeader*>(partials);
        if (slot == 0 && tid == 0) {
            hdr->rem[xcd] = (int32_t)plan.rem;
            hdr->S[xcd] = (int32_t)plan.S;
        }
        if (has_slice && slice_part == 0 && tid < 64) {  // decode by a whole wave
            TailTile tt;
            ts.decode(slice_lin, tt.row0, tt.row_end, tt.e, tt.n0);
            if (tid == 0) hdr->tile[xcd][slot / plan.S] = tt;
        }
    }
    if (nunits == 0) return;  // uniform per block
    auto unit_lin = [&](int u) { return u < (int)nw ? plan.chunk0 + slot + (uint32_t)u * nslots : slice_lin; };
    auto unit_kb = [&](int u) { return u < (int)nw ? 0 : slice_kb; };
    // K-grouped: the expert of a tile and its column range, read with scalar loads (a vector load
    // would be followed by a wait that also drains the DMAs in flight)
    const __attribute__((address_space(4))) int32_t* kg_poff = (const __attribute__((address_space(4))) int32_t*)kg.poff;
    auto kg_expert = [&](uint32_t lin) {
        int64_t row0, row_end;
        int e, n0;
        ts.decode(lin, row0, row_end, e, n0);
        return (int)(row0 / kg.m_per_e);
    };
    auto unit_ke = [&](int u) {
        if constexpr (KG) {
            const int ex = kg_expert(unit_lin(u));
            return (kg_poff[ex + 1] - kg_poff[ex]) / BK;
        } else {
            return u < (int)nw ? nk : slice_ke;
        }
    };

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t n_b_rows = GATED ? 2 * (int64_t)n_out : n_out;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)lds;

    // DMA q of this wave: LDS rows (q * 4 + wave) * 8 + [0, 8); rows 0-255 token tile, then the weights
    // (SwiGLU: BN / 2 gate rows, then the matching up rows)
    int voff[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int R = (q * 4 + wave) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz8(R);
        const int row = q < BM / 32 ? R : ((GATED && q >= QUP) ? R - BM - BN / 2 : R - BM);
        voff[q] = row * (KG ? (int)kg.ld : K) * 2 + c * 16;
    }
    // K not a multiple of BK (KT): the weight chunks of the last stage past K read as zeros. A lane's
    // chunk is the same in every DMA (swz8 of rows 32 q + 8 wave + lane / 8 does not depend on q).
    const int tor = KT && ((lane & 7) ^ swz8(wave * 8 + (lane >> 3))) * 8 >= K - (nk - 1) * BK ? (int)0x80000000 : 0;
    i32x4 ra, rb0, rb1;
    auto set_dma_tile = [&](uint32_t lin) {
        int64_t row0, row_end;
        int e, n0;
        ts.decode(lin, row0, row_end, e, n0);
        const int64_t a_rows = row_end - row0 < BM ? row_end - row0 : BM;
        if constexpr (KG) {  // rows m0 .. m0 + 255 of the expert, columns from its K offset
            const int ex = (int)(row0 / kg.m_per_e);
            const int64_t m0 = row0 - (int64_t)ex * kg.m_per_e;
            const int k0 = kg_poff[ex], kn = kg_poff[ex + 1] - k0;
            const int bcols = n_out - n0 < BN ? n_out - n0 : BN;
            ra = make_rsrc(A + m0 * kg.ld + k0, (uint32_t)(((int64_t)(BM - 1) * kg.ld + kn) * 2));
            rb0 = make_rsrc(B + (int64_t)n0 * kg.ld + k0, (uint32_t)(((int64_t)(bcols - 1) * kg.ld + kn) * 2));
            rb1 = rb0;
            return;
        }
        if (GA) {  // gathered token rows: the descriptor spans A, the row offsets follow the tile
            ra = make_rsrc(A, a_bytes);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                voff[q] = gathered_voff_uniform<8>(gather, row0, row_end, (q * 4 + wave) * 8, K);
            }
        } else {
            ra = make_rsrc(A + row0 * K, (uint32_t)(a_rows * K * 2));
        }
        const uint16_t* Bg = B + (int64_t)e * n_b_rows * K;
        const int bn_part = GATED ? BN / 2 : BN;
        const int bcols = n_out - n0 < bn_part ? n_out - n0 : bn_part;
        rb0 = make_rsrc(Bg + (int64_t)n0 * K, (uint32_t)((int64_t)bcols * K * 2));
        rb1 = make_rsrc(Bg + (int64_t)(GATED ? n_out + n0 : n0) * K, (uint32_t)((int64_t)bcols * K * 2));
    };

    // fragment rows: row block base + lane % 32, whose swizzle is that of lane % 32 (the bases are
    // multiples of 32)
    int a_off[TM], b_off[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a_off[i] = (wm * 128 + i * 32 + (lane & 31)) * BK;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int jj = j < TNO ? j : j - TNO;
        b_off[j] = (BM + (GATED && j >= TNO ? BN / 2 : 0) + wn * WTNO + jj * 32 + (lane & 31)) * BK;
    }
    const int fsw = swz8(lane & 31);
    const int khalf = lane >> 5;

    floatx16 acc[TM][TN];
    bf16x8 fa[2][TM], fb[2][TN];

#define PW_DMA(slot_, ks_, q_)                                                                            \
    dma16(lds_base + (slot_) * STAGE_BYTES + ((q_) * 4 + wave) * 1024,                                    \
          (KT && (q_) >= BM / 32 && (ks_) == nk - 1) ? (voff[q_] | tor) : voff[q_],                       \
          (q_) < BM / 32 ? ra : ((GATED && (q_) >= QUP) ? rb1 : rb0), (ks_) * (BK * 2));
    // fragment n (in MFMA use order: fa0, fb0..fb[TN-1], fa1..fa3) of 16-wide K step kk_ into buffer b_
#define PW_READ(b_, kk_, slot_, n_)                                                                       \
    {                                                                                                     \
        const uint16_t* L_ = lds + (slot_) * STAGE_ELEMS;                                                 \
        const int c_ = (kk_) * 2 + khalf;                                                                 \
        if ((n_) == 0 || (n_) > TN) {                                                                     \
            const int i_ = (n_) == 0 ? 0 : (n_) - TN;                                                     \
            fa[b_][i_] = *reinterpret_cast<const bf16x8*>(L_ + a_off[i_] + ((c_ ^ fsw) << 3));            \
        } else {                                                                                          \
            const int j_ = (n_) - 1;                                                                      \
            fb[b_][j_] = *reinterpret_cast<const bf16x8*>(L_ + b_off[j_] + ((c_ ^ fsw) << 3));            \
        }                                                                                                 \
    }
    // the compiler selects one register file for every MFMA accumulator of a kernel, so the ones kept in
    // VGPRs are multiplied through inline asm (their hazards are covered where they are zeroed and read)
#define PW_MMA(b_, t_)                                                                                    \
    if ((t_) % TN < NAG)                                                                                  \
        acc[(t_) / TN][(t_) % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                              \
            fb[b_][(t_) % TN], fa[b_][(t_) / TN], acc[(t_) / TN][(t_) % TN], 0, 0, 0);                    \
    else                                                                                                  \
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"                                            \
                     : "+v"(acc[(t_) / TN][(t_) % TN])                                                    \
                     : "v"(fb[b_][(t_) % TN]), "v"(fa[b_][(t_) / TN]));

    int dma_u = 0;
    set_dma_tile(unit_lin(0));
    int w_ks = unit_kb(0), w_ke = unit_ke(0);
    // past the block's last stage the DMAs go on with zero-range descriptors into the free slot
    auto dma_advance = [&]() {
        if (++w_ks == w_ke) {
            if (dma_u + 1 < nunits) {
                ++dma_u;
                set_dma_tile(unit_lin(dma_u));
                w_ks = unit_kb(dma_u);
                w_ke = unit_ke(dma_u);
            } else {
                ra = make_rsrc(A, 0);
                rb0 = ra;
                rb1 = ra;
            }
        }
    };
#pragma unroll
    for (int q = 0; q < NQ; ++q) PW_DMA(0, w_ks, q)
    dma_advance();
    wait_vm<0>();
    lds_barrier();
#pragma unroll
    for (int n = 0; n < NF; ++n) PW_READ(0, 0, 0, n)
    __builtin_amdgcn_sched_barrier(0);

    int r_slot = 0;
    // one stage: K steps 0 and 1 with the next stage's NQ DMAs after their odd MFMAs and the following
    // step's fragment reads after their even ones, step 2 with the reads of step 3, step 3: WB MFMAs,
    // the wait for the next stage's DMAs and the stage barrier, the rest with the reads of the next
    // stage's first step
#define PW_STAGE                                                                                          \
    {                                                                                                     \
        const int n_slot = r_slot ^ 1;                                                                    \
        _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                                  \
            PW_MMA(0, t)                                                                                  \
            if ((t & 1) && (t >> 1) < NQ / 2) PW_DMA(n_slot, w_ks, t >> 1)                                \
            if ((t & 1) == 0 && (t >> 1) < NF) PW_READ(1, 1, r_slot, t >> 1)                              \
            __builtin_amdgcn_sched_barrier(0);                                                            \
        }                                                                                                 \
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                                \
        __builtin_amdgcn_sched_barrier(0);                                                                \
        _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                                  \
            PW_MMA(1, t)                                                                                  \
            if ((t & 1) && (t >> 1) < NQ - NQ / 2) PW_DMA(n_slot, w_ks, NQ / 2 + (t >> 1))                \
            if ((t & 1) == 0 && (t >> 1) < NF) PW_READ(0, 2, r_slot, t >> 1)                              \
            __builtin_amdgcn_sched_barrier(0);                                                            \
        }                                                                                                 \
        dma_advance();                                                                                    \
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                                \
        __builtin_amdgcn_sched_barrier(0);                                                                \
        _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                                  \
            PW_MMA(0, t)                                                                                  \
            if ((t & 1) == 0 && (t >> 1) < NF) PW_READ(1, 3, r_slot, t >> 1)                              \
            __builtin_amdgcn_sched_barrier(0);                                                            \
        }                                                                                                 \
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                                \
        __builtin_amdgcn_sched_barrier(0);                                                                \
        _Pragma("unroll") for (int t = 0; t < WB; ++t) PW_MMA(1, t)                                       \
        __builtin_amdgcn_sched_barrier(0);                                                                \
        wait_vm<0>();                                                                                     \
        lds_barrier();                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                                \
        _Pragma("unroll") for (int t = WB; t < NT; ++t) {                                                 \
            PW_MMA(1, t)                                                                                  \
            if (t - WB < NF) PW_READ(0, 0, n_slot, t - WB)                                                \
            __builtin_amdgcn_sched_barrier(0);                                                            \
        }                                                                                                 \
        r_slot = n_slot;                                                                                  \
    }
    for (int u = 0; u < nunits; ++u) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        if constexpr (NAG < TN) asm volatile("s_nop 4" ::: "memory");  // VALU writes before MFMA reads
        const int ns = unit_ke(u) - unit_kb(u);
        for (int st = 0; st < ns; ++st) PW_STAGE
        // an MFMA's result is read by VALU instructions only some cycles after it issues
        if constexpr (NAG < TN) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        if (u < (int)nw) {
            int64_t row0, row_end;
            int e, n0;
            ts.decode(unit_lin(u), row0, row_end, e, n0);
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                store_block<EPI, TN, true, NAG>(acc[i], row0 + wm * 128 + i * 32 + (ln & 31), row_end, e,
                                           n0 + wn * WTNO, ln, C, bias, n_out);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            float* pb = partials;
            int ln = lane;
            asm volatile("" : "+s"(pb), "+v"(ln));
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                floatx4* dst = partial_at<2, TN>(pb, xcd * nslots + slot, wm * 4 + ((i >> 1) | (wn << 1)));
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v4 = 0; v4 < 4; ++v4)
                        *as_global(dst + (((i & 1) * TN + j) * 4 + v4) * 64 + ln) =
                            floatx4{acc_read<NAG>(j, acc[i][j][4 * v4]), acc_read<NAG>(j, acc[i][j][4 * v4 + 1]),
                                    acc_read<NAG>(j, acc[i][j][4 * v4 + 2]), acc_read<NAG>(j, acc[i][j][4 * v4 + 3])};
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm<0>();  // no DMA may land in LDS after the block has left the CU
#undef PW_STAGE
#undef PW_DMA
#undef PW_READ
#undef PW_MMA
}

// Tail of gemm_bf16_persistent_kernel: sums the S fp32 partial tiles of each split tail tile in
// slice order and applies the epilogue. One thread per group of 4 consecutive output features of
// one token (gate and up together for SwiGLU); block b covers XCD b % 8, tail tile (b / 8) / CH and
// chunk (b / 8) % CH of that tile's groups (launch: 8 * nslots * CH blocks of 256 threads, nslots
// the GEMM's blocks per XCD). Tile coordinates come from the header the GEMM wrote; R128 is the
// GEMM's tile layout.
template <int EPI, int TN = 4>
constexpr int tail_chunks() {
    return 8 * 2 * (EPI == EPI_SWIGLU ? TN / 2 : TN) * 4 * 64 / 256;  // (wave, i, j, v4, lane) groups / 256
}
template <int EPI, bool R128, int TN = 4>
__global__ __launch_bounds__(256) void gemm_bf16_tail_kernel(const float* __restrict__ partials,
                                                             const uint16_t* __restrict__ bias,
                                                             uint16_t* __restrict__ C, int n_out, int nslots) {
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int TM = 2, TNO = GATED ? TN / 2 : TN, WTNO = TNO * 32;
    constexpr int CH = tail_chunks<EPI, TN>();
    const TailHeader* hdr = reinterpret_cast<const TailHeader*>(partials);
    // work item b = (t * CH + ch) * 8 + xcd over every slot the GEMM could have split; the few that
    // hold a tail tile are the low ones, and a grid-stride loop over them launches far fewer blocks
    // than one block per item
    for (int b = blockIdx.x; b < 8 * nslots * CH; b += gridDim.x) {
        const int xcd = b & 7;
        const int t = (b >> 3) / CH, ch = (b >> 3) % CH;
        const int S = hdr->S[xcd];
        // the GEMM splits only when rem * S <= nslots, so every slot read below is one it wrote
        if (S < 2 || t >= hdr->rem[xcd] || t >= nslots || (t + 1) * S > nslots) continue;
        const TailTile tt = hdr->tile[xcd][t];
        const int gid = ch * 256 + threadIdx.x;  // group id: lane fastest, then v4, j, i, wave
        const int lane = gid & 63, v4 = (gid >> 6) & 3;
        const int j = (gid >> 8) % TNO, i = ((gid >> 8) / TNO) % TM, wave = (gid >> 8) / (TNO * TM);
        const int grp = wave >> 2, wig = wave & 3, wm = wig & 1, wn = wig >> 1;
        floatx4 z = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
        for (int sidx = 0; sidx < S; ++sidx) {
            const floatx4* src =
                partial_at<TM, TN>(const_cast<float*>(partials), xcd * nslots + t * S + sidx, wave);
            z += src[((i * TN + j) * 4 + v4) * 64 + lane];
            if (GATED) u += src[((i * TN + j + TNO) * 4 + v4) * 64 + lane];
        }
        const int64_t row = tt.row0 + wave_row_base<R128>(grp, wm) + i * 32 + (lane & 31);
        const int f0 = tt.n0 + wave_feat_base<R128, WTNO>(grp, wn) + j * 32 + 8 * v4 + 4 * (lane >> 5);
        if (row >= tt.row_end || f0 >= n_out) continue;
        if (EPI == EPI_F32) {
            *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(C) + row * n_out + f0) = z;
            continue;
        }
        float o[4];
        if (GATED) {
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = z[c] * __builtin_amdgcn_rcpf(1.0f + __expf(-z[c])) * u[c];
        } else {
            float bc[4] = {0.f, 0.f, 0.f, 0.f};
            if (bias != nullptr) {
                const uint2 bb = *reinterpret_cast<const uint2*>(bias + (int64_t)tt.e * n_out + f0);
                bc[0] = __uint_as_float(bb.x << 16);
                bc[1] = __uint_as_float(bb.x & 0xffff0000u);
                bc[2] = __uint_as_float(bb.y << 16);
                bc[3] = __uint_as_float(bb.y & 0xffff0000u);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = EPI == EPI_GELU_BIAS ? gelu_f(z[c] + bc[c]) : z[c] + bc[c];
        }
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
        *reinterpret_cast<uint2*>(C + row * n_out + f0) = pk;
    }
}

// Blocks of the tail pass: one per possible work item (8 XCDs x slots x chunks), at most 2048; the
// kernel loops over the rest.
unsigned tail_grid(unsigned gemm_grid, int chunks) {
    const unsigned items = gemm_grid * (unsigned)chunks;
    return items < 2048u ? items : 2048u;
}

// Blocks of the persistent GEMM: the CU count in whole XCD rounds, at most 8 * kMaxSlotsPerXcd.
int persistent_grid_cap() {
    const int cap = (device_cu_count() / 8) * 8;
    return cap < 8 * kMaxSlotsPerXcd ? cap : 8 * kMaxSlotsPerXcd;
}

// Bytes of the partial buffer the bf16 grouped GEMM may use (header + one 256 x 256 fp32 tile per
// block).
size_t gemm_partials_bytes(int dtype) {
    if (dtype != MOE_BF16) return 0;
    return kTailHeaderBytes + (size_t)persistent_grid_cap() * kPartialFloats * sizeof(float);
}

template <int GM, int D, bool R128>
void launch_bf16_persistent(int epi, const void* A, const void* B, const void* bias, void* C,
                            const int32_t* offsets, int e_begin, int n_groups, int64_t max_rows, int64_t dense_rows,
                            int n_out, int K, float* partials, hipStream_t s, const int32_t* gather,
                            uint32_t a_bytes) {
    constexpr int bm = R128 ? 128 : 256;
    const int bno = (epi == EPI_SWIGLU ? 128 : 256) * (R128 ? 2 : 1);
    const int64_t m_tiles = offsets ? (max_rows + bm - 1) / bm + n_groups : (dense_rows + bm - 1) / bm;
    const int64_t tiles = m_tiles * ((n_out + bno - 1) / bno);
    if (tiles <= 0) return;
    const int64_t cap = persistent_grid_cap();
    const int64_t want = ((tiles + 7) / 8) * 8;
    // a dense product with fewer tiles than CUs takes every CU anyway when it may split along K
    const unsigned grid = (unsigned)(want < cap && (offsets || !partials) ? want : cap);
    // a dense product whose tiles fill whole rounds needs no tail pass
    if (!offsets && tiles % grid == 0) partials = nullptr;
    const auto a = static_cast<const uint16_t*>(A);
    const auto b = static_cast<const uint16_t*>(B);
    const auto bi = static_cast<const uint16_t*>(bias);
    auto c = static_cast<uint16_t*>(C);
#define MOE_PERSIST_GA(EPI_, GA_)                                                                          \
    {                                                                                                     \
        if (K % 32)                                                                                       \
            gemm_bf16_persistent_kernel<EPI_, GM, D, true, R128, GA_><<<grid, 512, 0, s>>>(               \
                a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out, K, partials, gather, a_bytes);  \
        else                                                                                              \
            gemm_bf16_persistent_kernel<EPI_, GM, D, false, R128, GA_><<<grid, 512, 0, s>>>(              \
                a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out, K, partials, gather, a_bytes);  \
    }
    // gathered rows only on the up projections (gated or GELU epilogues); the others build without
    // the gather path
#define MOE_PERSIST(EPI_)                                                                                 \
    {                                                                                                     \
        if constexpr (EPI_ == EPI_SWIGLU || EPI_ == EPI_GELU_BIAS) {                                      \
            if (gather) MOE_PERSIST_GA(EPI_, true)                                                        \
            else MOE_PERSIST_GA(EPI_, false)                                                              \
        } else {                                                                                          \
            MOE_PERSIST_GA(EPI_, false)                                                                   \
        }                                                                                                 \
        if (partials)                                                                                     \
            gemm_bf16_tail_kernel<EPI_, R128><<<tail_grid(grid, tail_chunks<EPI_>()), 256, 0, s>>>(        \
                partials, bi, c, n_out, (int)(grid / 8));                                                 \
    }
    if (epi == EPI_SWIGLU) MOE_PERSIST(EPI_SWIGLU)
    else if (epi == EPI_GELU_BIAS) MOE_PERSIST(EPI_GELU_BIAS)
    else if (epi == EPI_F32) MOE_PERSIST(EPI_F32)
    else MOE_PERSIST(EPI_BIAS)
#undef MOE_PERSIST
#undef MOE_PERSIST_GA
}

template <int GM, int BN>
void launch_bf16_wide(int epi, const void* A, const void* B, const void* bias, void* C, const int32_t* offsets,
                    int e_begin, int n_groups, int64_t max_rows, int64_t dense_rows, int n_out, int K, float* partials,
                    hipStream_t s, const int32_t* gather, uint32_t a_bytes) {
    const int bno = epi == EPI_SWIGLU ? BN / 2 : BN;
    const int64_t m_tiles = offsets ? (max_rows + 255) / 256 + n_groups : (dense_rows + 255) / 256;
    const int64_t tiles = m_tiles * ((n_out + bno - 1) / bno);
    if (tiles <= 0) return;
    const int64_t cap = persistent_grid_cap();
    const int64_t want = ((tiles + 7) / 8) * 8;
    const unsigned grid = (unsigned)(want < cap && (offsets || !partials) ? want : cap);
    if (!offsets && tiles % grid == 0) partials = nullptr;
    const auto a = static_cast<const uint16_t*>(A);
    const auto b = static_cast<const uint16_t*>(B);
    const auto bi = static_cast<const uint16_t*>(bias);
    auto c = static_cast<uint16_t*>(C);
#define MOE_WIDE_GA(EPI_, GA_)                                                                             \
    {                                                                                                     \
        if (K % 64)                                                                                       \
            gemm_bf16_wide_kernel<EPI_, GM, true, GA_, BN, false><<<grid, 256, 0, s>>>(                   \
                a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out, K, partials, gather, a_bytes,   \
                KgArgs{nullptr, 0, 0});                                                                   \
        else                                                                                              \
            gemm_bf16_wide_kernel<EPI_, GM, false, GA_, BN, false><<<grid, 256, 0, s>>>(                  \
                a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out, K, partials, gather, a_bytes,   \
                KgArgs{nullptr, 0, 0});                                                                   \
    }
#define MOE_WIDE(EPI_)                                                                                      \
    {                                                                                                     \
        if constexpr (EPI_ == EPI_SWIGLU || EPI_ == EPI_GELU_BIAS) {                                      \
            if (gather) MOE_WIDE_GA(EPI_, true)                                                           \
            else MOE_WIDE_GA(EPI_, false)                                                                 \
        } else {                                                                                          \
            MOE_WIDE_GA(EPI_, false)                                                                      \
        }                                                                                                 \
        if (partials)                                                                                     \
            gemm_bf16_tail_kernel<EPI_, false, BN / 64>                                                   \
                <<<tail_grid(grid, tail_chunks<EPI_, BN / 64>()), 256, 0, s>>>(partials, bi, c, n_out,    \
                                                                               (int)(grid / 8));          \
    }
    if (epi == EPI_SWIGLU) MOE_WIDE(EPI_SWIGLU)
    else if (epi == EPI_GELU_BIAS) MOE_WIDE(EPI_GELU_BIAS)
    else if (epi == EPI_F32) MOE_WIDE(EPI_F32)
    else MOE_WIDE(EPI_BIAS)
#undef MOE_WIDE
#undef MOE_WIDE_GA
}

void launch_wgrad_kgrouped(const void* AT, const void* BT, float* C, const int32_t* poff, int E, int m_per_e,
                           int n_out, int64_t ld, hipStream_t s) {
    const int64_t rows = (int64_t)E * m_per_e;
    const int64_t tiles = (rows / 256) * ((n_out + 383) / 384);
    if (tiles <= 0) return;
    const int64_t cap = persistent_grid_cap();
    const int64_t want = ((tiles + 7) / 8) * 8;
    const unsigned grid = (unsigned)(want < cap ? want : cap);
    gemm_bf16_wide_kernel<EPI_F32, 8, false, false, 384, true><<<grid, 256, 0, s>>>(
        static_cast<const uint16_t*>(AT), static_cast<const uint16_t*>(BT), nullptr, reinterpret_cast<uint16_t*>(C),
        nullptr, 0, 0, rows, n_out, 64, nullptr, nullptr, 0u, KgArgs{poff, ld, m_per_e});
}

// fp32 path (SIMT, 64 x 64 output tile, 4 x 4 per thread, sequential fp32 FMA over K).
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                       const float* __restrict__ bias, float* __restrict__ C,
                                                       const int32_t* __restrict__ offsets, int e_begin,
                                                       int n_groups, int64_t dense_rows, int n_out, int K) {
    constexpr int BM = 64, BNO = 64, BK = 16;
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int NB = GATED ? 2 : 1;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[NB][BK][BNO + 4];
    __shared__ int s_ts[1025];
    __shared__ int s_wave[4];
    if (offsets) build_schedule<BM, 256>(offsets, e_begin, n_groups, s_ts, s_wave);
    const TileCoord tc = decode_tile<BM, BNO, 8>(offsets, s_ts, e_begin, n_groups, dense_rows, n_out);
    if (!tc.valid) return;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t last_row = tc.row_end - 1;
    const int64_t n_b_rows = GATED ? 2 * (int64_t)n_out : n_out;
    const float* Bg = B + (int64_t)tc.e * n_b_rows * K;
    const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row (0..63), k quad
    const int64_t arow = tc.row0 + lr <= last_row ? tc.row0 + lr : last_row;
    const int bcol = tc.n0 + lr < n_out ? tc.n0 + lr : n_out - 1;
    float acc[NB][4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kk = k0 + lk + q;
            As[lk + q][lr] = kk < K ? A[arow * K + kk] : 0.f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                Bs[nb][lk + q][lr] = kk < K ? Bg[((int64_t)nb * n_out + bcol) * K + kk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[NB][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int j = 0; j < 4; ++j) b[nb][j] = Bs[nb][kk][tx * 4 + j];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[nb][i][j] = fmaf(a[i], b[nb][j], acc[nb][i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = tc.row0 + ty * 4 + i;
        if (row >= tc.row_end) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = tc.n0 + tx * 4 + j;
            if (col >= n_out) continue;
            float out;
            if (EPI == EPI_SWIGLU) {
                out = silu_f(acc[0][i][j]) * acc[NB - 1][i][j];
            } else {
                const float bc = bias != nullptr ? bias[(int64_t)tc.e * n_out + col] : 0.f;
                out = EPI == EPI_GELU_BIAS ? gelu_f(acc[0][i][j] + bc) : acc[0][i][j] + bc;
            }
            C[row * n_out + col] = out;
        }
    }
}

GemmPlan plan_gemm(int dtype, int64_t rows_per_group_hint, int n_out, int K) {
    (void)n_out;
    (void)K;
    GemmPlan p;
    // bf16: groups of a few dozen rows (decode batches) are bound by streaming their weights, which
    // 64-row tiles with a deep operand ring do better than the 256-row persistent tiles
    p.bm = dtype == MOE_BF16 ? (rows_per_group_hint <= kGemmSmallRowsMax ? 64 : 256) : 64;
    return p;
}

template <int BM, int BN, int NS, int GM>
void launch_bf16_tiles(int epi, const void* A, const void* B, const void* bias, void* C, const int32_t* offsets,
                       int e_begin, int n_groups, int64_t max_rows, int64_t dense_rows, int n_out, int K,
                       hipStream_t s, const int32_t* gather, uint32_t a_bytes) {
    const int bno = epi == EPI_SWIGLU ? BN / 2 : BN;
    const int64_t m_tiles = offsets ? (max_rows + BM - 1) / BM + n_groups : (dense_rows + BM - 1) / BM;
    const int64_t n_tiles = (n_out + bno - 1) / bno;
    const int64_t tiles = m_tiles * n_tiles;
    const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);  // whole XCD rounds
    const auto a = static_cast<const uint16_t*>(A);
    const auto b = static_cast<const uint16_t*>(B);
    const auto bi = static_cast<const uint16_t*>(bias);
    auto c = static_cast<uint16_t*>(C);
#define MOE_TILES(EPI_)                                                                                   \
    {                                                                                                     \
        if (K % 32)                                                                                       \
            gemm_bf16_kernel<BM, BN, EPI_, NS, GM, true><<<grid, 256, 0, s>>>(                            \
                a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out, K, gather, a_bytes);            \
        else                                                                                              \
            gemm_bf16_kernel<BM, BN, EPI_, NS, GM, false><<<grid, 256, 0, s>>>(                           \
                a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out, K, gather, a_bytes);            \
    }
    if constexpr (BN >= 128) {  // a gated tile holds gate and up halves of at least 64 columns each
        if (epi == EPI_SWIGLU) {
            MOE_TILES(EPI_SWIGLU)
            return;
        }
    }
    if (epi == EPI_GELU_BIAS) MOE_TILES(EPI_GELU_BIAS)
    else if (epi == EPI_F32) MOE_TILES(EPI_F32)
    else MOE_TILES(EPI_BIAS)
#undef MOE_TILES
}

void launch_grouped_gemm(int dtype, int epi, int bm, const void* A, const void* B, const void* bias, void* C,
                         const int32_t* offsets, int e_begin, int n_groups, int64_t max_rows, int64_t dense_rows,
                         int n_out, int K, float* partials, hipStream_t s, const int32_t* gather, int64_t a_rows) {
    const uint32_t a_bytes = gather ? (uint32_t)(a_rows * K * 2) : 0u;
    if (dtype == MOE_BF16) {
        if (bm == 128 && offsets == nullptr && epi == EPI_F32 &&
            ((dense_rows + 127) / 128) * ((n_out + 127) / 128) >= device_cu_count()) {
            // dense fp32-output products with a short output (the wide routers' logits, x [T, d] x
            // [3 Epad, d]) whose 128 x 128 tiles fill the CUs: one tile per block, two blocks per CU,
            // no K split, so no fp32 partial tiles are written and summed. Measured on the routes:
            // Qwen3-shaped (384 tiles, K = 2048) 86.4 -> 72.4 us; the DeepSeek-shaped one (192 tiles,
            // K = 7168) was slower this way (94.5 against 125.4 us) and keeps the persistent kernel's
            // K split.
            launch_bf16_tiles<128, 128, 4, 8>(epi, A, B, bias, C, offsets, e_begin, n_groups, max_rows, dense_rows,
                                              n_out, K, s, gather, a_bytes);
            return;
        }
        if (bm == 64 && offsets != nullptr && epi != EPI_F32) {
            // small groups: 64-row x 128-column tiles with a 6-stage LDS ring (72 KB, two blocks per CU).
            // Measured on the decode batch: 128-wide panels beat 256-wide ones (more tiles to spread
            // over the CUs), and two blocks per CU with 6 stages beat one block with 9 or 13. A
            // non-gated projection with fewer than 512 such tiles (the down projection of a decode
            // batch: 8 experts x 32 panels) takes 64-wide panels with an 8-stage ring (64 KB), so each
            // CU holds two blocks: 260 -> 253-257 us there.
            if (epi != EPI_SWIGLU && (int64_t)n_groups * ((n_out + 127) / 128) < 512) {
                launch_bf16_tiles<64, 64, 8, 8>(epi, A, B, bias, C, offsets, e_begin, n_groups, max_rows, dense_rows,
                                                n_out, K, s, gather, a_bytes);
                return;
            }
            launch_bf16_tiles<64, 128, 6, 8>(epi, A, B, bias, C, offsets, e_begin, n_groups, max_rows, dense_rows,
                                             n_out, K, s, gather, a_bytes);
            return;
        }
        // expert groups averaging at least kGemmWideRows rows (kGemmWideRowsLongK over a K of at least
        // kGemmWideMinK) take the four-wave wide-K kernel; smaller groups and dense products keep the
        // eight-wave kernel, whose deeper ring streams weights better
        const int64_t ng = n_groups > 0 ? n_groups : 1;
        if (offsets != nullptr &&
            (max_rows >= kGemmWideRows * ng || (K >= kGemmWideMinK && max_rows >= kGemmWideRowsLongK * ng)))
        {
            if (kGemmWideBN > 256 && n_groups <= kRegSchedGroups)
                launch_bf16_wide<8, kGemmWideBN>(epi, A, B, bias, C, offsets, e_begin, n_groups, max_rows,
                                                 dense_rows, n_out, K, partials, s, gather, a_bytes);
            else
                launch_bf16_wide<8, 256>(epi, A, B, bias, C, offsets, e_begin, n_groups, max_rows, dense_rows,
                                         n_out, K, partials, s, gather, a_bytes);
        }
        else if (offsets != nullptr && max_rows <= kGemmR128Rows * ng)
            launch_bf16_persistent<8, 2, true>(epi, A, B, bias, C, offsets, e_begin, n_groups, max_rows,
                                               dense_rows, n_out, K, partials, s, gather, a_bytes);
        else
            launch_bf16_persistent<8, 3, false>(epi, A, B, bias, C, offsets, e_begin, n_groups, max_rows,
                                                dense_rows, n_out, K, partials, s, gather, a_bytes);
        return;
    }
    const int64_t m_tiles = offsets ? (max_rows + 63) / 64 + n_groups : (dense_rows + 63) / 64;
    const int64_t tiles = m_tiles * ((n_out + 63) / 64);
    const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
    const auto a = static_cast<const float*>(A);
    const auto b = static_cast<const float*>(B);
    const auto bi = static_cast<const float*>(bias);
    auto c = static_cast<float*>(C);
    if (epi == EPI_SWIGLU)
        gemm_f32_kernel<EPI_SWIGLU><<<grid, 256, 0, s>>>(a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out, K);
    else if (epi == EPI_GELU_BIAS)
        gemm_f32_kernel<EPI_GELU_BIAS><<<grid, 256, 0, s>>>(a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out,
                                                            K);
    else
        gemm_f32_kernel<EPI_BIAS><<<grid, 256, 0, s>>>(a, b, bi, c, offsets, e_begin, n_groups, dense_rows, n_out, K);
}

}  // namespace moe

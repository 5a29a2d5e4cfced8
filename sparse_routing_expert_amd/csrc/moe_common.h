// Device helpers shared by the libmoe kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bfloat16 <-> fp32. The narrowing conversion is the hardware round-to-nearest-even
// (v_cvt_pk_bf16_f32); widening is exact.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
// 8 bf16 held in a 128-bit vector -> 8 floats (element i is bits [16i, 16i+16)).
__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Wave-wide reductions (all 64 lanes participate; every lane receives the same result). Inside each
// 16-lane row, DPP moves combine lanes (quad xor 1, quad xor 2, row rotate 4, row rotate 8); lane 0
// of every row then holds (Q0 + Q1) + (Q2 + Q3) of its row's quads, and the four row results are
// read into scalars and combined as (R0 + R1) + (R2 + R3): a fixed order, so results are
// deterministic, with no LDS round trip.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppRor4>(v);
    v += dpp_f32<kDppRor8>(v);
    return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppRor4>(v));
    v = fmaxf(v, dpp_f32<kDppRor8>(v));
    return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<kDppXor1>(v));
    v = max_u64(v, dpp_u64<kDppXor2>(v));
    v = max_u64(v, dpp_u64<kDppRor4>(v));
    v = max_u64(v, dpp_u64<kDppRor8>(v));
    return max_u64(max_u64(lane_u64(v, 0), lane_u64(v, 16)), max_u64(lane_u64(v, 32), lane_u64(v, 48)));
}

// Reductions over each 16-lane DPP row (xor 1, xor 2 inside quads, then the half-row and row
// mirrors). Every step pairs each lane with a partner that holds the mirrored operand, so by the
// commutativity of + and max every lane of a row ends with the same bits: ((q0 + q1) + (q2 + q3))
// over the quad sums.
constexpr int kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    return v;
}
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    return v;
}
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<kDppXor1>(v));
    v = max_u64(v, dpp_u64<kDppXor2>(v));
    v = max_u64(v, dpp_u64<kDppHalfMirror>(v));
    v = max_u64(v, dpp_u64<kDppMirror>(v));
    return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace moe

namespace moe {

// Exclusive prefix sum over a block of exactly 1024 threads (16 waves). `s_wave` is LDS scratch
// of 17 ints. Returns the exclusive prefix of `v`; *total receives the block-wide sum.
__device__ __forceinline__ int block1024_excl_scan(int v, int* s_wave, int* total) {
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int n = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += n;
    }
    if (lane == kWave - 1) s_wave[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < 16; ++w) {
            int c = s_wave[w];
            s_wave[w] = run;
            run += c;
        }
        s_wave[16] = run;
    }
    __syncthreads();
    *total = s_wave[16];
    return s_wave[wave] + inc - v;
}

}  // namespace moe

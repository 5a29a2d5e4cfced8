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

// Wave-wide reductions (all 64 lanes participate; every lane receives the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
        uint64_t w = ((uint64_t)hi << 32) | lo;
        v = w > v ? w : v;
    }
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

// dsa_device.hpp -- device helpers shared by the libdsa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
    return __uint_as_float(packed & 0xffff0000u);
}

// binary32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Four OCP e4m3 codes (one dword) -> four bf16 (two dwords). Exact: every e4m3 value is a
// bf16 value. gfx950 converts two codes per instruction.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t codes) {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
    u32x2 r;
    r.x = __builtin_bit_cast(uint32_t, lo);
    r.y = __builtin_bit_cast(uint32_t, hi);
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// e^x through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Float -> unsigned key that orders like the float (finite and +-inf); -0 maps like +0.
__device__ __forceinline__ uint32_t ordered_key(float f) {
    if (f == 0.0f) f = 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// ------------------------------------------------------------------ block scans
// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, at most 1024).
// `scratch` must hold NT/64 + 1 ints. Returns the exclusive prefix; *total gets the sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int *total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    if (lane == kWave - 1) scratch[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        constexpr int NW = NT / kWave;
        int x = lane < NW ? scratch[lane] : 0;
        int xi = x;
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            int o = __shfl_up(xi, d, kWave);
            if (lane >= d) xi += o;
        }
        if (lane < NW) scratch[lane] = xi - x;
        if (lane == NW - 1) scratch[NW] = xi;
    }
    __syncthreads();
    int excl = scratch[wave] + inc - v;
    *total = scratch[NT / kWave];
    __syncthreads();
    return excl;
}

template <int NT>
__device__ __forceinline__ int block_sum(int v, int *scratch) {
    int total;
    (void)block_exclusive_scan<NT>(v, scratch, &total);
    return total;
}

}  // namespace dsa

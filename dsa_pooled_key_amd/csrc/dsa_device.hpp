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

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
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

// Eight e4m3 codes (two dwords) -> eight bf16 (four dwords), exact.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    const u32x2 a = e4m3x4_to_bf16x4(lo), b = e4m3x4_to_bf16x4(hi);
    return u32x4{a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef short __attribute__((ext_vector_type(4))) i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// gfx950 LDS transpose read of 16-bit elements (ds_read_b64_tr_b16). Each lane addresses
// 8 bytes (4 elements) of LDS; within every group of 16 lanes, result lane i, element e is
// element i%4 of the 8 bytes addressed by lane 4*e + i/4 of the same group.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t *lds_ptr) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lds_ptr));
    return __builtin_bit_cast(u32x2, v);
}

typedef int __attribute__((ext_vector_type(2))) i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// gfx950 LDS transpose read of 8-bit elements (ds_read_b64_tr_b8). Each lane addresses
// 8 bytes; within every group of 16 lanes, result lane i, byte e is byte i%8 of the 8 bytes
// addressed by lane 2*e + i/8 of the same group.
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t *lds_ptr) {
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(lds_ptr));
    return __builtin_bit_cast(u32x2, v);
}

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

// Inverse of ordered_key (for keys of finite floats and +-inf).
__device__ __forceinline__ float ordered_key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
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

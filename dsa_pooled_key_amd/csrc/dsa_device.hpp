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

// gfx950 lane swaps (v_permlane16_swap / v_permlane32_swap) applied to two copies of v: the
// pair holds v of rows {0,0,2,2} and {1,1,3,3} (16-lane rows), or of lanes 0-31 and 32-63 each
// repeated twice, so op(first, second) reduces across lanes l and l ^ 16 (or l ^ 32) in two
// VALU instructions and no LDS trip.
__device__ __forceinline__ float max_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ------------------------------------------------------------------ HBM -> LDS copies
// One 16-byte-a-lane global -> LDS copy (global_load_lds_dwordx4): lane l's 16 bytes land
// at lds_base + 16*l. Issued as inline assembly without a memory clobber, so the compiler
// neither orders nearby LDS reads behind it nor waits for it: it only writes a stage that no
// code reads before the explicit vmcnt wait and block barrier that publish it (loads complete
// in order, so the compiler's own waits for other loads stay correct).
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "m0");
}

// Same for 4 bytes a lane (global_load_lds_dword): lane l's dword lands at lds_base + 4*l.
__device__ __forceinline__ void dma4(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "m0");
}

// A raw buffer resource over [base, base + bytes): accesses past the end are dropped (loads
// return 0). Word 3 is the usual gfx9 setting for untyped access (32-bit data format, which
// only typed accesses read; no swizzle, no thread-id offset).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)(p);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
// The builtin form lets the compiler's own wait insertion see these waits.
template <int N>
__device__ __forceinline__ void wait_vm() {  // at most N vector-memory loads outstanding
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ------------------------------------------------------------------ wave primitives (DPP)
// Cross-lane steps through DPP (the VALU reads a neighbour lane's register in the same
// instruction), not through LDS: GFX9 controls quad_perm, row_shr:n, row_ror:n (rows are 16
// lanes) and row_bcast:15/31. All of these are used with the whole wave active.
namespace dpp {
constexpr int kXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142;  // lane 15 of each row to the whole next row
constexpr int kRowBcast31 = 0x143;  // lane 31 to rows 2 and 3
}  // namespace dpp

// v of the DPP source lane; 0 where the control gives no source or the row is masked off.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele in each row, then the row carries).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
    v += dpp_or_zero<dpp::kRowShr1>(v);
    v += dpp_or_zero<dpp::kRowShr2>(v);
    v += dpp_or_zero<dpp::kRowShr4>(v);
    v += dpp_or_zero<dpp::kRowShr8>(v);
    v += dpp_or_zero<dpp::kRowBcast15, 0xa>(v);
    v += dpp_or_zero<dpp::kRowBcast31, 0xc>(v);
    return v;
}

// Reductions over the 64 lanes: a butterfly inside each row, then the four row results
// (lanes 0, 16, 32, 48) read into scalars. The result is wave-uniform.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
    v = op(v, dpp_mov<dpp::kXor1>(v));
    v = op(v, dpp_mov<dpp::kXor2>(v));
    v = op(v, dpp_mov<dpp::kRowRor4>(v));
    v = op(v, dpp_mov<dpp::kRowRor8>(v));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return op(op(a, b), op(c, d));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x + y; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}

// ------------------------------------------------------------------ block scans
// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, at most 1024).
// `scratch` must hold NT/64 + 1 ints. Returns the exclusive prefix; *total gets the sum.
// Each wave scans in registers and publishes its total; after one barrier every thread adds
// the totals of the waves before its own. A trailing barrier lets the caller reuse scratch.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int *total) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int inc = (int)wave_incl_sum((uint32_t)v);
    if (lane == kWave - 1) scratch[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int x = scratch[w];
        before += w < wave ? x : 0;
        all += x;
    }
    *total = all;
    __syncthreads();
    return before + inc - v;
}

template <int NT>
__device__ __forceinline__ int block_sum(int v, int *scratch) {
    int total;
    (void)block_exclusive_scan<NT>(v, scratch, &total);
    return total;
}

}  // namespace dsa

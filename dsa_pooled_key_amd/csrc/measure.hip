// measure.hip -- measurement kernels: what the part delivers, beside its nominal figures.
//
// None of these is a step of the method. They give the rates the decode and prefill kernels
// are compared with:
//   stream_read  the HBM read rate of the simplest access pattern (every byte read once, 16
//                bytes a lane, four loads in flight per lane, blocks striding over the whole
//                buffer); each block folds what it read into one word (XOR), so the loads
//                cannot be dropped;
//   empty        a kernel that does nothing, for the gap between dependent launches (a graph of
//                many of them, replayed);
//   mfma_rate    each wave runs four independent chains of one MFMA shape back to back, so the
//                matrix unit never waits on a result; the sum of the accumulators is stored
//                once per thread, so the chains cannot be dropped.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ buf, size_t n16,
                                                               uint32_t *__restrict__ sink) {
    uint32_t acc = 0u;
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc = wave_reduce_u32(acc, [](uint32_t a, uint32_t b) { return a ^ b; });
    if ((threadIdx.x & (kWave - 1)) == 0) atomicXor(sink, acc);
}

__global__ __launch_bounds__(kWave) void empty_kernel() {}

typedef __attribute__((ext_vector_type(8))) int i32x8;

// Shapes: 0 = v_mfma_f32_32x32x16_bf16, 1 = v_mfma_f32_16x16x32_bf16,
// 2 = v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 operands (scales 1).
template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(int iters, float *__restrict__ out) {
    u32x4 a;
    a.x = 0x3f803f80u + threadIdx.x;  // bf16 pairs near 1 (varied per lane)
    a.y = 0x3f803f81u;
    a.z = 0x3f813f80u;
    a.w = 0x3f803f82u;
    // A different B operand for each chain: with equal operands and equal starting values the
    // compiler merges the chains and rotates one result through register moves every round.
    u32x4 b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) b[k] = u32x4{a.x ^ (0x00010000u << k), a.y, a.z + k, a.w};
    const i32x8 fa = {0x38383838, 0x38383839, 0x3838383a, 0x3838383b, 0x3939393a, 0x3a3a3a3b,
                      0x3b3b3b3c, (int)(0x30303030u + threadIdx.x)};
    i32x8 fb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        fb[k] = i32x8{0x30303030 + k, 0x30303031, 0x30303032, 0x30303033, 0x31313131, 0x32323232,
                      0x33333333, 0x34343434};
    float s = 0.0f;
    if constexpr (KIND == 0) {
        f32x16 d0 = {}, d1 = {}, d2 = {}, d3 = {};
        for (int it = 0; it < iters; ++it) {
            d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b[0]), d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b[1]), d1, 0, 0, 0);
            d2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b[2]), d2, 0, 0, 0);
            d3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b[3]), d3, 0, 0, 0);
        }
        s = d0[0] + d1[5] + d2[10] + d3[15];
    } else {
        // Each chain alternates between two accumulators (x = mfma(y), y = mfma(x)): the
        // compiler keeps a 16x16 MFMA's destination apart from its accumulator input, and with
        // one accumulator per chain it would copy the result back every round.
        f32x4 x[4], y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] = f32x4{(float)k, (float)k, (float)k, (float)k};
        for (int it = 0; it < iters; it += 2) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (KIND == 1)
                    x[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b[k]), y[k], 0, 0, 0);
                else
                    x[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[k], y[k], 0, 0, 0, 127, 0, 127);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (KIND == 1)
                    y[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b[k]), x[k], 0, 0, 0);
                else
                    y[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[k], x[k], 0, 0, 0, 127, 0, 127);
            }
        }
        const f32x4 c0 = y[0], c1 = y[1], c2 = y[2], c3 = y[3];
        s = c0[0] + c1[1] + c2[2] + c3[3];
    }
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int blocks,
                              hipStream_t stream) {
    if (bytes < 16) return hipSuccess;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_empty(int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(kWave), 0, stream);
    return hipGetLastError();
}

hipError_t launch_mfma_rate(int kind, int blocks, int iters, float *out, hipStream_t stream) {
    switch (kind) {
    case 0:
        hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(blocks), dim3(kThreads), 0, stream, iters, out);
        break;
    case 1:
        hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(blocks), dim3(kThreads), 0, stream, iters, out);
        break;
    default:
        hipLaunchKernelGGL(mfma_rate_kernel<2>, dim3(blocks), dim3(kThreads), 0, stream, iters, out);
        break;
    }
    return hipGetLastError();
}

}  // namespace dsa

// compact_pools.hip -- ascending list of valid pools per sequence.
//
// mod.rs names dsa_compact_pools between pooling and scoring; here it is a stable stream
// compaction: one 1024-thread block per sequence walks the validity row in chunks of 16,384
// pools (16 per thread), a block prefix sum places each valid id in an LDS stage, the stage is
// stored as one contiguous run, and the tail of the id row is filled with -1. Reads P bytes
// and writes 4*P bytes per sequence.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = 16;
constexpr int kChunk = kThreads * kPer;  // pools per pass

__global__ __launch_bounds__(kThreads) void compact_pools_kernel(int P,
                                                                 const uint8_t *__restrict__ pv,
                                                                 int32_t *__restrict__ ids,
                                                                 int32_t *__restrict__ n_valid) {
    __shared__ int scratch[kThreads / kWave + 1];
    __shared__ int32_t stage[kChunk];
    const long long b = blockIdx.x;
    const uint8_t *row = pv + b * P;
    int32_t *out = ids + b * P;
    const bool vec = ((reinterpret_cast<uintptr_t>(row) | (uintptr_t)P) & 15) == 0;
    int base = 0;
    for (int c0 = 0; c0 < P; c0 += kChunk) {
        const int p0 = c0 + threadIdx.x * kPer;
        uint32_t bits = 0;
        if (vec && p0 + kPer <= P) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(row + p0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if ((w[j >> 2] >> ((j & 3) * 8)) & 0xffu) bits |= 1u << j;
        } else {
            for (int j = 0; j < kPer; ++j)
                if (p0 + j < P && row[p0 + j]) bits |= 1u << j;
        }
        int total;
        int off = block_exclusive_scan<kThreads>(__popc(bits), scratch, &total);
        // Stage the chunk's ids in pool order, then store them as one contiguous run.
        while (bits) {
            const int j = __ffs(bits) - 1;
            bits &= bits - 1;
            stage[off++] = p0 + j;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < total; i += kThreads) out[base + i] = stage[i];
        __syncthreads();
        base += total;
    }
    for (int p = base + threadIdx.x; p < P; p += kThreads) out[p] = -1;
    if (threadIdx.x == 0) n_valid[b] = base;
}

}  // namespace

hipError_t launch_compact_pools(int B, int P, const uint8_t *pool_valid, int32_t *ids,
                                int32_t *n_valid, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(compact_pools_kernel, dim3(B), dim3(kThreads), 0, stream, P, pool_valid,
                       ids, n_valid);
    return hipGetLastError();
}

}  // namespace dsa

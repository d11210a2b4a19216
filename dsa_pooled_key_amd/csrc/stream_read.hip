// stream_read.hip -- a plain streaming read of a device buffer, for measurement only.
//
// Not a step of the method: it gives the HBM read rate this part achieves with the simplest
// access pattern (every byte read once, 16 bytes a lane, four loads in flight per lane, blocks
// striding over the whole buffer), the figure the decode kernels' bandwidth is compared with
// beside the nominal peak. Each block folds what it read into one word (XOR), so the loads
// cannot be dropped.
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

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int blocks,
                              hipStream_t stream) {
    if (bytes < 16) return hipSuccess;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace dsa

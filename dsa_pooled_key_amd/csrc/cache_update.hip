// cache_update.hip -- decode-time upkeep of the indexer cache.
//
// mod.rs, Glm5NextDsaKernels: `k_norm` is a LayerNorm with a bias applied in place to bf16
// rows (x, weight, bias, rows, dim, eps); `indexer_store` copies the staged indexer row to
// a device-side position and marks it valid; `write_geom` derives the selector geometry on
// the device from seq_len, so a captured graph replays over the live context. The pool a
// new token completes is handled beside the pooling kernel (kpool_compress.hip), which it
// shares.
//
// All three are small and latency-bound: per row 2D bytes in and out (LayerNorm), per
// sequence 4D bytes plus a flag (store), 12 bytes (geometry).
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

// G = D/8 consecutive lanes own one row (8 values each, one 16-byte load and store); a wave
// holds 64/G rows. Mean and variance (two passes over the registers, f32) meet through
// lane swaps inside the group.
__global__ __launch_bounds__(256) void layer_norm_kernel(long long rows, int D, int G,
                                                         uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ weight,
                                                         const uint16_t *__restrict__ bias,
                                                         float eps) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long row = gid / G;
    if (row >= rows) return;  // whole groups
    const int d0 = (int)(gid - row * G) * 8;
    uint16_t *px = x + row * D + d0;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(px);
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
    float f[8];
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        f[c] = (c & 1) ? bf16_hi(vw[c >> 1]) : bf16_lo(vw[c >> 1]);
        sum += f[c];
    }
    for (int m = G >> 1; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, kWave);
    const float mean = sum / (float)D;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) sq += (f[c] - mean) * (f[c] - mean);
    for (int m = G >> 1; m >= 1; m >>= 1) sq += __shfl_xor(sq, m, kWave);
    const float inv = 1.0f / sqrtf(sq / (float)D + eps);
    const u32x4 w = *reinterpret_cast<const u32x4 *>(weight + d0);
    const u32x4 bb = *reinterpret_cast<const u32x4 *>(bias + d0);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w}, bw[4] = {bb.x, bb.y, bb.z, bb.w};
    float y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float wc = (c & 1) ? bf16_hi(ww[c >> 1]) : bf16_lo(ww[c >> 1]);
        const float bc = (c & 1) ? bf16_hi(bw[c >> 1]) : bf16_lo(bw[c >> 1]);
        y[c] = (f[c] - mean) * inv * wc + bc;
    }
    *reinterpret_cast<u32x4 *>(px) = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                           pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
}

// Block b copies sequence b's staged key and gate rows (16 bytes a thread) to position
// pos[b] and marks it valid; a position outside [0, S) stores nothing.
__global__ __launch_bounds__(64) void indexer_store_kernel(int S, int D,
                                                           const int32_t *__restrict__ pos,
                                                           const uint16_t *__restrict__ k_row,
                                                           const uint16_t *__restrict__ gate_row,
                                                           uint16_t *__restrict__ k_cache,
                                                           uint16_t *__restrict__ gate_cache,
                                                           uint8_t *__restrict__ valid) {
    const long long b = blockIdx.x;
    const int t = pos[b];
    if (t < 0 || t >= S) return;
    const long long dst = (b * S + t) * D;
    for (int d0 = threadIdx.x * 8; d0 < D; d0 += 64 * 8) {
        *reinterpret_cast<u32x4 *>(k_cache + dst + d0) =
            *reinterpret_cast<const u32x4 *>(k_row + b * D + d0);
        *reinterpret_cast<u32x4 *>(gate_cache + dst + d0) =
            *reinterpret_cast<const u32x4 *>(gate_row + b * D + d0);
    }
    if (threadIdx.x == 0) valid[b * S + t] = 1;
}

__global__ __launch_bounds__(256) void write_geom_kernel(int B, const int32_t *__restrict__ seq_len,
                                                         int32_t *__restrict__ row_seq,
                                                         int32_t *__restrict__ row_pos) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    row_seq[b] = b;
    row_pos[b] = seq_len[b] - 1;
}

}  // namespace

hipError_t launch_layer_norm(long long rows, int D, uint16_t *x, const uint16_t *weight,
                             const uint16_t *bias, float eps, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int G = D / 8;
    const long long threads = rows * G;
    hipLaunchKernelGGL(layer_norm_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, rows, D, G, x, weight, bias, eps);
    return hipGetLastError();
}

hipError_t launch_indexer_store(int B, int S, int D, const int32_t *pos, const uint16_t *k_row,
                                const uint16_t *gate_row, uint16_t *k_cache, uint16_t *gate_cache,
                                uint8_t *valid, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(indexer_store_kernel, dim3(B), dim3(64), 0, stream, S, D, pos, k_row,
                       gate_row, k_cache, gate_cache, valid);
    return hipGetLastError();
}

hipError_t launch_write_geom(int B, const int32_t *seq_len, int32_t *row_seq, int32_t *row_pos,
                             hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(write_geom_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, B, seq_len,
                       row_seq, row_pos);
    return hipGetLastError();
}

}  // namespace dsa

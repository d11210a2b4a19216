// kpool_compress.hip -- pooled indexer keys.
//
// mod.rs, "Shape of the pipeline" and "Checkpoint and kernel facts": a pool is index_kpool
// consecutive token slots starting at first_key; per channel the slot weights are a softmax
// over the slots of gate + ape, the pooled key is the weighted sum of the slot keys, and the
// pool is valid only when every slot is. The page's own kernel keeps the logits in an
// 8-float register array; here each thread owns 8 channels of one pool and keeps all
// KP x 8 logits in registers, so one pool row is written by D/8 threads with 16-byte
// stores, and consecutive threads read consecutive 16-byte pieces of each token row.
//
// HBM-bound: per pool KP*D*2 (k) + KP*D*2 (gate) + KP (valid) bytes in, D*2 + 1 out.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

template <int KP>
__global__ __launch_bounds__(256) void kpool_compress_kernel(
    int S, int D, int first_key, int P, long long n_pools, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ gate, const float *__restrict__ ape,
    const uint8_t *__restrict__ valid, uint16_t *__restrict__ pool_keys,
    uint8_t *__restrict__ pool_valid) {
    const int tpp = D >> 3;  // threads per pool
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long pool = gid / tpp;
    if (pool >= n_pools) return;
    const int d0 = (int)(gid - pool * tpp) * 8;
    const long long b = pool / P;
    const long long p = pool - b * P;
    const long long t0 = (long long)first_key + p * KP;
    const long long row0 = b * S + t0;

    float x[KP][8];
    float mx[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) mx[c] = -INFINITY;
#pragma unroll
    for (int s = 0; s < KP; ++s) {
        const u32x4 g = *reinterpret_cast<const u32x4 *>(gate + (row0 + s) * D + d0);
        const f32x4 a0 = *reinterpret_cast<const f32x4 *>(ape + s * D + d0);
        const f32x4 a1 = *reinterpret_cast<const f32x4 *>(ape + s * D + d0 + 4);
        const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
        const float aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float gv = (c & 1) ? bf16_hi(gw[c >> 1]) : bf16_lo(gw[c >> 1]);
            x[s][c] = gv + aw[c];
            mx[c] = fmaxf(mx[c], x[s][c]);
        }
    }
    float den[8], acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        den[c] = 0.0f;
        acc[c] = 0.0f;
    }
#pragma unroll
    for (int s = 0; s < KP; ++s) {
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(k + (row0 + s) * D + d0);
        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float e = fast_exp(x[s][c] - mx[c]);
            const float kc = (c & 1) ? bf16_hi(kw[c >> 1]) : bf16_lo(kw[c >> 1]);
            den[c] += e;
            acc[c] += e * kc;
        }
    }
    u32x4 o;
    o.x = pack_bf16x2(acc[0] / den[0], acc[1] / den[1]);
    o.y = pack_bf16x2(acc[2] / den[2], acc[3] / den[3]);
    o.z = pack_bf16x2(acc[4] / den[4], acc[5] / den[5]);
    o.w = pack_bf16x2(acc[6] / den[6], acc[7] / den[7]);
    *reinterpret_cast<u32x4 *>(pool_keys + pool * D + d0) = o;
    if (d0 == 0) {
        int ok = 1;
#pragma unroll
        for (int s = 0; s < KP; ++s) ok &= valid[row0 + s] != 0;
        pool_valid[pool] = (uint8_t)ok;
    }
}

template <int KP>
hipError_t launch_kp(int B, int S, int D, int first_key, int P, const uint16_t *k,
                     const uint16_t *gate, const float *ape, const uint8_t *valid,
                     uint16_t *pool_keys, uint8_t *pool_valid, hipStream_t stream) {
    const long long n_pools = (long long)B * P;
    const long long threads = n_pools * (D / 8);
    const long long blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(kpool_compress_kernel<KP>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       S, D, first_key, P, n_pools, k, gate, ape, valid, pool_keys, pool_valid);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kpool_compress(int B, int S, int D, int KP, int first_key, int P,
                                 const uint16_t *k, const uint16_t *gate, const float *ape,
                                 const uint8_t *valid, uint16_t *pool_keys, uint8_t *pool_valid,
                                 hipStream_t stream) {
    if ((long long)B * P == 0) return hipSuccess;
    switch (KP) {
#define DSA_KP_CASE(n) \
    case n: return launch_kp<n>(B, S, D, first_key, P, k, gate, ape, valid, pool_keys, pool_valid, stream);
        DSA_KP_CASE(1) DSA_KP_CASE(2) DSA_KP_CASE(3) DSA_KP_CASE(4)
        DSA_KP_CASE(5) DSA_KP_CASE(6) DSA_KP_CASE(7) DSA_KP_CASE(8)
#undef DSA_KP_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa

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
// HBM-bound: per pool KP*D*2 (k) + KP*D*2 (gate) + KP (valid) bytes in, D*2 + 1 out (D + 4 + 1
// with fp8 output).
//
// The fp8 writers (the stored format of fp8 pooled keys and latent rows): per row the scale is
// amax/448 and each value is stored as e4m3(value / scale), rounded to nearest even and
// saturating; both divisions are IEEE single precision.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

// Four values -> four OCP e4m3 codes in one dword (value i in byte i), nearest-even; the
// values are clamped to +-448 first, which makes the conversion saturating.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    auto cl = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
    return (uint32_t)w;
}

// Per-row fp8 scale of a row whose largest magnitude is amax: amax / 448 (1 for a zero row).
__device__ __forceinline__ float fp8_row_scale(float amax) {
    return amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
}

// Channels d0 .. d0+7 of pool p of sequence b: the softmax over the KP slots of gate + ape
// weighting the slot keys, rounded to bf16 (four packed pairs).
template <int KP>
__device__ __forceinline__ u32x4 pool_channels8(int S, int D, int first_key, long long b,
                                                long long p, int d0,
                                                const uint16_t *__restrict__ k,
                                                const uint16_t *__restrict__ gate,
                                                const float *__restrict__ ape) {
    const long long row0 = b * S + (long long)first_key + p * KP;
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
    return o;
}

// Stores channels d0 .. d0+7 of pool row `pool` (index into [B*P]): bf16, or (FP8OUT) fp8
// quantized per pool row -- scale s = amax/448 over the row's D values, whose D/8 threads
// are consecutive lanes (tpp of them, a power of two) and meet through lane swaps.
template <bool FP8OUT>
__device__ __forceinline__ void store_pool_channels8(const u32x4 &o, long long pool, int D, int d0,
                                                     int tpp, void *__restrict__ pool_keys,
                                                     float *__restrict__ key_scales) {
    if constexpr (!FP8OUT) {
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(pool_keys) + pool * D + d0) = o;
    } else {
        const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
        float vb[8];
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            vb[c] = (c & 1) ? bf16_hi(ow[c >> 1]) : bf16_lo(ow[c >> 1]);
            amax = fmaxf(amax, fabsf(vb[c]));
        }
        for (int m = tpp >> 1; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
        const float sc = fp8_row_scale(amax);
        float q[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) q[c] = __fdiv_rn(vb[c], sc);
        *reinterpret_cast<u32x2 *>(static_cast<uint8_t *>(pool_keys) + pool * D + d0) =
            u32x2{e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7])};
        if (d0 == 0) key_scales[pool] = sc;
    }
}

// FP8OUT: the pooled key is rounded to bf16 as usual and then stored as fp8 (see above).
template <int KP, bool FP8OUT = false>
__global__ __launch_bounds__(256) void kpool_compress_kernel(
    int S, int D, int first_key, int P, long long n_pools, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ gate, const float *__restrict__ ape,
    const uint8_t *__restrict__ valid, void *__restrict__ pool_keys,
    float *__restrict__ key_scales, uint8_t *__restrict__ pool_valid) {
    const int tpp = D >> 3;  // threads per pool
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long pool = gid / tpp;
    if (pool >= n_pools) return;  // whole groups of tpp lanes
    const int d0 = (int)(gid - pool * tpp) * 8;
    const long long b = pool / P;
    const long long p = pool - b * P;
    const u32x4 o = pool_channels8<KP>(S, D, first_key, b, p, d0, k, gate, ape);
    store_pool_channels8<FP8OUT>(o, pool, D, d0, tpp, pool_keys, key_scales);
    if (d0 == 0) {
        const long long row0 = b * S + (long long)first_key + p * KP;
        int ok = 1;
#pragma unroll
        for (int s = 0; s < KP; ++s) ok &= valid[row0 + s] != 0;
        pool_valid[pool] = (uint8_t)ok;
    }
}

// Decode-time upkeep: block b (one wave) looks at the token just stored at pos[b]; when it
// is the last slot of pool p (pos >= first_key, (pos - first_key + 1) % KP == 0, p < P), the
// wave computes that pool exactly as kpool_compress_kernel does (lanes < D/8, 8 channels
// each), sets its validity and, if valid, appends p to the compacted ids unless the list
// already ends at p or beyond (so a repeated call changes nothing).
template <int KP, bool FP8OUT>
__global__ __launch_bounds__(64) void pool_append_kernel(
    int S, int D, int first_key, int P, const int32_t *__restrict__ pos,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ gate,
    const float *__restrict__ ape, const uint8_t *__restrict__ valid,
    void *__restrict__ pool_keys, float *__restrict__ key_scales,
    uint8_t *__restrict__ pool_valid, int32_t *__restrict__ ids, int32_t *__restrict__ n_valid) {
    const long long b = blockIdx.x;
    const int t = pos[b];
    if (t < first_key || t >= S || (t - first_key + 1) % KP != 0) return;
    const long long p = (t - first_key + 1) / KP - 1;
    if (p >= P) return;
    const int tpp = D >> 3;
    const int lane = threadIdx.x;
    if (lane < tpp) {
        const int d0 = lane * 8;
        const u32x4 o = pool_channels8<KP>(S, D, first_key, b, p, d0, k, gate, ape);
        store_pool_channels8<FP8OUT>(o, b * P + p, D, d0, tpp, pool_keys, key_scales);
    }
    if (lane == 0) {
        const long long row0 = b * S + (long long)first_key + p * KP;
        int ok = 1;
#pragma unroll
        for (int s = 0; s < KP; ++s) ok &= valid[row0 + s] != 0;
        pool_valid[b * P + p] = (uint8_t)ok;
        const int n = n_valid[b];
        if (ok && n >= 0 && n < P && (n == 0 || ids[b * P + n - 1] < p)) {
            ids[b * P + n] = (int32_t)p;
            n_valid[b] = n + 1;
        }
    }
}

template <int KP>
hipError_t launch_kp(int B, int S, int D, int first_key, int P, const uint16_t *k,
                     const uint16_t *gate, const float *ape, const uint8_t *valid,
                     void *pool_keys, float *key_scales, uint8_t *pool_valid, hipStream_t stream) {
    const long long n_pools = (long long)B * P;
    const long long threads = n_pools * (D / 8);
    const long long blocks = (threads + 255) / 256;
    if (key_scales)
        hipLaunchKernelGGL((kpool_compress_kernel<KP, true>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, S, D, first_key, P, n_pools, k, gate, ape, valid, pool_keys,
                           key_scales, pool_valid);
    else
        hipLaunchKernelGGL((kpool_compress_kernel<KP, false>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, S, D, first_key, P, n_pools, k, gate, ape, valid, pool_keys,
                           key_scales, pool_valid);
    return hipGetLastError();
}

// One wave per row of n values (n a multiple of 8, at most 64 * 8 * CH): lane l holds
// values 8(64c + l) .. +7 of chunk c < CH in registers between the amax reduction and the
// encoding, so the row is read once. Each wave takes RPW rows and requests all of them before
// reducing any, to keep more loads in flight.
template <bool F32SRC, int CH, int RPW>
__global__ __launch_bounds__(256) void quantize_rows_kernel(long long rows, int n,
                                                            const void *__restrict__ src,
                                                            uint8_t *__restrict__ codes,
                                                            float *__restrict__ scales) {
    const long long row0 = ((long long)blockIdx.x * 4 + threadIdx.x / kWave) * RPW;
    if (row0 >= rows) return;  // the whole wave
    const int lane = threadIdx.x & (kWave - 1);
    float v[RPW][CH][8];
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const long long row = row0 + j;
            const int i0 = (c * kWave + lane) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[j][c][e] = 0.0f;
            if (row < rows && i0 < n) {
                if constexpr (F32SRC) {
                    const float *p = static_cast<const float *>(src) + row * n + i0;
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
                    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
                    v[j][c][0] = a.x; v[j][c][1] = a.y; v[j][c][2] = a.z; v[j][c][3] = a.w;
                    v[j][c][4] = b.x; v[j][c][5] = b.y; v[j][c][6] = b.z; v[j][c][7] = b.w;
                } else {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(
                        static_cast<const uint16_t *>(src) + row * n + i0);
                    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[j][c][e] = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
                }
            }
        }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        const long long row = row0 + j;
        if (row >= rows) break;  // uniform over the wave
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][c][e]));
        // magnitudes are non-negative, so they order like their bit patterns
        amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));
        const float sc = fp8_row_scale(amax);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i0 = (c * kWave + lane) * 8;
            if (i0 < n) {
                float q[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = __fdiv_rn(v[j][c][e], sc);
                *reinterpret_cast<u32x2 *>(codes + row * n + i0) =
                    u32x2{e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7])};
            }
        }
        if (lane == 0) scales[row] = sc;
    }
}

template <bool F32SRC, int CH>
hipError_t launch_quant(long long rows, int n, const void *src, uint8_t *codes, float *scales,
                        hipStream_t stream) {
    constexpr int kRpw = CH == 1 ? 2 : 1;
    const long long waves = (rows + kRpw - 1) / kRpw;
    hipLaunchKernelGGL((quantize_rows_kernel<F32SRC, CH, kRpw>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(256), 0, stream, rows, n, src, codes, scales);
    return hipGetLastError();
}

template <bool F32SRC>
hipError_t launch_quant_any(long long rows, int n, const void *src, uint8_t *codes, float *scales,
                            hipStream_t stream) {
    if (n <= 512) return launch_quant<F32SRC, 1>(rows, n, src, codes, scales, stream);
    if (n <= 1024) return launch_quant<F32SRC, 2>(rows, n, src, codes, scales, stream);
    if (n <= 2048) return launch_quant<F32SRC, 4>(rows, n, src, codes, scales, stream);
    return launch_quant<F32SRC, 8>(rows, n, src, codes, scales, stream);
}

}  // namespace

hipError_t launch_kpool_compress(int B, int S, int D, int KP, int first_key, int P,
                                 const uint16_t *k, const uint16_t *gate, const float *ape,
                                 const uint8_t *valid, void *pool_keys, float *key_scales,
                                 uint8_t *pool_valid, hipStream_t stream) {
    if ((long long)B * P == 0) return hipSuccess;
    switch (KP) {
#define DSA_KP_CASE(n) \
    case n: return launch_kp<n>(B, S, D, first_key, P, k, gate, ape, valid, pool_keys, key_scales, \
                                pool_valid, stream);
        DSA_KP_CASE(1) DSA_KP_CASE(2) DSA_KP_CASE(3) DSA_KP_CASE(4)
        DSA_KP_CASE(5) DSA_KP_CASE(6) DSA_KP_CASE(7) DSA_KP_CASE(8)
#undef DSA_KP_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_pool_append(int B, int S, int D, int KP, int first_key, int P,
                              const int32_t *pos, const uint16_t *k, const uint16_t *gate,
                              const float *ape, const uint8_t *valid, void *pool_keys,
                              float *key_scales, uint8_t *pool_valid, int32_t *ids,
                              int32_t *n_valid, hipStream_t stream) {
    if (B == 0 || P == 0) return hipSuccess;
#define DSA_APPEND(n, f8)                                                                        \
    hipLaunchKernelGGL((pool_append_kernel<n, f8>), dim3(B), dim3(64), 0, stream, S, D, first_key, P, \
                       pos, k, gate, ape, valid, pool_keys, key_scales, pool_valid, ids, n_valid)
#define DSA_APPEND_KP(n)                              \
    case n:                                           \
        if (key_scales) DSA_APPEND(n, true);          \
        else DSA_APPEND(n, false);                    \
        break;
    switch (KP) {
        DSA_APPEND_KP(1) DSA_APPEND_KP(2) DSA_APPEND_KP(3) DSA_APPEND_KP(4)
        DSA_APPEND_KP(5) DSA_APPEND_KP(6) DSA_APPEND_KP(7) DSA_APPEND_KP(8)
        default: return hipErrorInvalidValue;
    }
#undef DSA_APPEND_KP
#undef DSA_APPEND
    return hipGetLastError();
}

hipError_t launch_quantize_rows(long long rows, int n, const void *src, bool f32_src,
                                uint8_t *codes, float *scales, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    return f32_src ? launch_quant_any<true>(rows, n, src, codes, scales, stream)
                   : launch_quant_any<false>(rows, n, src, codes, scales, stream);
}

}  // namespace dsa

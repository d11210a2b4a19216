// masked_attn.hip -- the dense masked-attention cross-check of the sparse decode.
//
// mod.rs, Glm5NextDsaKernels::{topk_to_mask, mla_masked_attn} and MASKED_ATTN_MAX_KEYS: the
// selection is turned into a [Q, S] token mask, and a dense attention that stages the whole
// [S] f32 score row in on-chip memory attends over every masked token. It is a second,
// independent route to the sparse decode's result (only checks call it). The pages' kernel
// holds 12,288 scores in 48 KB; a gfx950 block holds DSA_MASKED_ATTN_MAX_KEYS = 32,768 in
// 128 KiB of its 160 KiB LDS.
//
// mla_masked_attn: block (r, h), 4 waves. The mask row is first copied into the LDS score
// row as markers. Scores: wave w walks the positions in chunks of 64 (a ballot of the
// markers), and for each masked token its lanes take 8
// channels each of the latent row (one 1 KiB bf16 or 512 B fp8 row per wave load, up to
// eight tokens in flight), a DPP sum gives the logit. Then a block max and sum, and the
// output: wave w owns channels 128w..128w+127 and walks the positions again, accumulating
// p_t * v_t for the masked ones. Latent rows are addressed as the sparse decode addresses
// them (contiguous b*S + t, or through the block table; absent rows are skipped).
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

constexpr int kC = 512;

// Positions [c0, c0 + kMaskChunk) of row r: cleared, marked from the row's token ids, written.
constexpr int kMaskChunk = 32768;
__global__ __launch_bounds__(256) void topk_to_mask_kernel(int W, int S,
                                                           const int32_t *__restrict__ token_ids,
                                                           uint8_t *__restrict__ mask) {
    __shared__ __attribute__((aligned(16))) uint8_t m[kMaskChunk];
    const long long r = blockIdx.x;
    const int c0 = blockIdx.y * kMaskChunk;
    const int n = min(kMaskChunk, S - c0);
    for (int i = threadIdx.x * 16; i < kMaskChunk; i += 256 * 16)
        *reinterpret_cast<u32x4 *>(&m[i]) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    for (int i = threadIdx.x; i < W; i += 256) {
        const int t = token_ids[r * W + i];
        if (t >= c0 && t < c0 + n) m[t - c0] = 1;
    }
    __syncthreads();
    uint8_t *dst = mask + r * S + c0;
    for (int i = threadIdx.x; i < n; i += 256) dst[i] = m[i];
}

template <bool FP8, bool PAGED>
__global__ __launch_bounds__(256) void masked_attn_kernel(
    int S, int H, int B, float sm_scale, const uint16_t *__restrict__ q_abs,
    const uint8_t *__restrict__ mask, const int32_t *__restrict__ row_seq,
    const void *__restrict__ kv, const float *__restrict__ kv_scales, long long kv_rows,
    const int32_t *__restrict__ block_table, int max_blocks, int block_size,
    float *__restrict__ out, float *__restrict__ lse) {
    __shared__ float sc[DSA_MASKED_ATTN_MAX_KEYS];
    __shared__ float red[2][4];
    const long long r = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int b = row_seq[r];
    const bool row_ok = b >= 0 && b < B;
    const uint8_t *mrow = mask + r * S;
    const uint8_t *kvb = static_cast<const uint8_t *>(kv);
    constexpr int RB = FP8 ? kC : 2 * kC;

    auto latent = [&](int t) -> long long {  // row of token t, or -1
        if (!row_ok) return -1;
        long long row;
        if constexpr (PAGED) {
            const int blk = t / block_size;
            if (blk >= max_blocks) return -1;
            const int pb = block_table[(long long)b * max_blocks + blk];
            if (pb < 0) return -1;
            row = (long long)pb * block_size + (t - blk * block_size);
        } else {
            row = (long long)b * S + t;
        }
        return row < kv_rows ? row : -1;
    };
    // Lane's 8 query channels 8*lane .. +7 (f32).
    float qf[8];
    {
        const u32x4 qv = *reinterpret_cast<const u32x4 *>(q_abs + ((r * H + h) * kC) + 8 * lane);
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) qf[c] = (c & 1) ? bf16_hi(qw[c >> 1]) : bf16_lo(qw[c >> 1]);
    }
    auto row_vals8 = [&](long long row, float (&v)[8]) {  // channels 8*lane .. +7 of a row
        if constexpr (FP8) {
            const u32x2 raw = *reinterpret_cast<const u32x2 *>(kvb + row * RB + 8 * lane);
            const u32x4 bf = e4m3x8_to_bf16x8(raw.x, raw.y);
            const uint32_t bw[4] = {bf.x, bf.y, bf.z, bf.w};
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] = (c & 1) ? bf16_hi(bw[c >> 1]) : bf16_lo(bw[c >> 1]);
        } else {
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(kvb + row * RB + 16 * lane);
            const uint32_t bw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] = (c & 1) ? bf16_hi(bw[c >> 1]) : bf16_lo(bw[c >> 1]);
        }
    };

    // ---- the mask row into the score row (+inf marks a masked slot, -inf the others), with
    // independent byte loads, so the scan below runs on LDS
#pragma unroll 8
    for (int t = tid; t < S; t += 256) sc[t] = mrow[t] != 0 ? INFINITY : -INFINITY;
    __syncthreads();
    // ---- scores: every masked position gets its logit (-inf when its latent row is absent);
    // a chunk's masked tokens go up to kBatch at a time, their row loads in flight together
    constexpr int kBatch = 8;
    for (int t0 = w * kWave; t0 < S; t0 += 4 * kWave) {
        const int t = t0 + lane;
        uint64_t bits = __ballot(t < S && sc[t] == INFINITY);
        while (bits != 0u) {
            int tt[kBatch];
            long long rw[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                tt[j] = -1;
                rw[j] = -1;
                if (bits != 0u) {
                    tt[j] = t0 + __builtin_ctzll(bits);
                    bits &= bits - 1u;
                    rw[j] = latent(tt[j]);
                }
            }
            float v[kBatch][8];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (rw[j] >= 0) row_vals8(rw[j], v[j]);
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (tt[j] >= 0 && rw[j] < 0 && lane == 0) sc[tt[j]] = -INFINITY;
                if (rw[j] < 0) continue;  // uniform: the whole wave takes the same token
                float d = 0.0f;
#pragma unroll
                for (int c = 0; c < 8; ++c) d += qf[c] * v[j][c];
                d += shfl_xor_f(d, 1);
                d += shfl_xor_f(d, 2);
                d += shfl_xor_f(d, 4);
                d += shfl_xor_f(d, 8);
                d += shfl_xor_f(d, 16);
                d += shfl_xor_f(d, 32);
                const float s = FP8 ? kv_scales[rw[j]] : 1.0f;
                if (lane == 0) sc[tt[j]] = sm_scale * (s * d);
            }
        }
    }
    __syncthreads();

    // ---- max and sum over the row
    float mx = -INFINITY;
    for (int t = tid; t < S; t += 256) mx = fmaxf(mx, sc[t]);
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, m));
    if (lane == 0) red[0][w] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    float sum = 0.0f;
    if (mx > -INFINITY)
        for (int t = tid; t < S; t += 256) sum += sc[t] > -INFINITY ? expf(sc[t] - mx) : 0.0f;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) sum += shfl_xor_f(sum, m);
    if (lane == 0) red[1][w] = sum;
    __syncthreads();
    sum = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);

    // ---- output: wave w owns channels 128w + 2*lane, +1
    float a0 = 0.0f, a1 = 0.0f;
    if (sum > 0.0f) {
        const float inv = 1.0f / sum;
        const int c = 128 * w + 2 * lane;
        for (int t0 = 0; t0 < S; t0 += kWave) {
            const int t = t0 + lane;
            uint64_t bits = __ballot(t < S && sc[t] > -INFINITY);
            while (bits != 0u) {
                int tt[kBatch];
                long long rw[kBatch];
                uint32_t raw[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    tt[j] = -1;
                    rw[j] = -1;
                    if (bits != 0u) {
                        tt[j] = t0 + __builtin_ctzll(bits);
                        bits &= bits - 1u;
                        rw[j] = latent(tt[j]);
                    }
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    raw[j] = 0u;
                    if (rw[j] >= 0) {
                        if constexpr (FP8)
                            raw[j] = *reinterpret_cast<const uint16_t *>(kvb + rw[j] * RB + c);
                        else
                            raw[j] = *reinterpret_cast<const uint32_t *>(kvb + rw[j] * RB + 2 * c);
                    }
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    if (rw[j] < 0) continue;
                    const float p = expf(sc[tt[j]] - mx) * inv * (FP8 ? kv_scales[rw[j]] : 1.0f);
                    float x0, x1;
                    if constexpr (FP8) {
                        const u32x2 bf = e4m3x4_to_bf16x4(raw[j]);
                        x0 = bf16_lo(bf.x);
                        x1 = bf16_hi(bf.x);
                    } else {
                        x0 = bf16_lo(raw[j]);
                        x1 = bf16_hi(raw[j]);
                    }
                    a0 += p * x0;
                    a1 += p * x1;
                }
            }
        }
    }
    float *o = out + (r * H + h) * kC + 128 * w + 2 * lane;
    o[0] = a0;
    o[1] = a1;
    if (lse != nullptr && tid == 0) lse[r * H + h] = sum > 0.0f ? mx + logf(sum) : -INFINITY;
}

}  // namespace

hipError_t launch_topk_to_mask(int Q, int W, int S, const int32_t *token_ids, uint8_t *mask,
                               hipStream_t stream) {
    if (Q == 0 || S == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_to_mask_kernel, dim3(Q, (S + kMaskChunk - 1) / kMaskChunk), dim3(256), 0,
                       stream, W, S, token_ids, mask);
    return hipGetLastError();
}

hipError_t launch_masked_attn(int Q, int H, int S, int B, float sm_scale, const uint16_t *q_abs,
                              const uint8_t *mask, const int32_t *row_seq, const void *kv,
                              bool kv_fp8, const float *kv_scales, int64_t kv_rows,
                              const int32_t *block_table, int max_blocks, int block_size,
                              float *out, float *lse, hipStream_t stream) {
    if (Q == 0 || H == 0) return hipSuccess;
    const dim3 grid(Q, H);
#define DSA_MASKED(f8, pg)                                                                          \
    hipLaunchKernelGGL((masked_attn_kernel<f8, pg>), grid, dim3(256), 0, stream, S, H, B, sm_scale, \
                       q_abs, mask, row_seq, kv, kv_scales, (long long)kv_rows, block_table,        \
                       max_blocks, block_size, out, lse)
    const bool paged = block_table != nullptr;
    if (kv_fp8) {
        if (paged) DSA_MASKED(true, true);
        else DSA_MASKED(true, false);
    } else {
        if (paged) DSA_MASKED(false, true);
        else DSA_MASKED(false, false);
    }
#undef DSA_MASKED
    return hipGetLastError();
}

}  // namespace dsa

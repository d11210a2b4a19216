// sparse_mla_decode.hip -- absorbed-query NoPE MLA attention over the selected tokens.
//
// build.rs, "The transforms" 1 and 3: the query is absorbed into the 512-wide latent and the
// output stays in latent space ([heads, kv_lora_rank]); mod.rs: NoPE, a 512-wide latent,
// attention restricted to the expanded token ids, and the serve path reads those tokens
// through a block table with no sequence-length-sized buffer.
//
// Keys and values are the same latent rows, so each 32-token tile is gathered once from
// HBM (bf16, or fp8 converted exactly to bf16 in registers), stored once in LDS as a
// [token][channel] bf16 tile, and read by both products:
//   S^T = K . Q^T  on v_mfma_f32_16x16x32_bf16: wave w computes 16 tokens x 16 heads over all
//                  512 channels; its query fragment (64 registers) stays resident.
//   O  += P . V    on v_mfma_f32_32x32x16_bf16: wave w owns 32 heads x 128 channels of the
//                  output accumulator (64 registers) and reads P (bf16) from LDS and V as
//                  16-bit elements down the token axis of the same tile.
// The softmax is online (running max and sum per head). The two waves that score the same
// 16 heads exchange their tile maxima through LDS; each keeps its own partial sum, combined
// at the end. For fp8 the per-token scale multiplies the logit and the probability, so no
// rounding beyond bf16 P is added.
//
// Split over tokens: block (r, s, g) takes token slots [s*L, s*L + L) of row r for head group
// g. With one split the block writes out and lse directly; with several it writes
// (max, sum, unnormalised O) to the workspace and mla_combine merges them.
//
// Bytes per selected token: 1024 (bf16) or 516 (fp8 + scale) of latent, 4 of token id.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

constexpr int kC = 512;
constexpr int kTile = 32;
constexpr int kThreads = 256;
constexpr int kKtStride = kC + 8;     // bf16 per tile row: 1040 B, shifts banks by 16 B a row
constexpr int kPStride = kTile + 8;   // bf16 per P row
constexpr int kPartFloats = 64 + 32 * kC;  // per (row, group, split): max[32], sum[32], O[32][512]

template <bool FP8, bool PAGED>
__global__ __launch_bounds__(kThreads) void sparse_mla_kernel(
    int W, int H, int B, int splits, int split_len, float sm_scale,
    const uint16_t *__restrict__ q_abs, const int32_t *__restrict__ token_ids,
    const int32_t *__restrict__ row_seq, const void *__restrict__ kv,
    const float *__restrict__ kv_scales, long long kv_rows, int S,
    const int32_t *__restrict__ block_table, int max_blocks, int block_size,
    float *__restrict__ out, float *__restrict__ lse, float *__restrict__ ws) {
    __shared__ __attribute__((aligned(16))) uint16_t kt[kTile * kKtStride];
    __shared__ __attribute__((aligned(16))) uint16_t pl[32 * kPStride];
    __shared__ float tok_scale[kTile];
    __shared__ int tok_ok[kTile];
    __shared__ float red[4][16];
    __shared__ float alpha_s[32];
    __shared__ float msum_s[32];
    __shared__ float lsum_s[32];
    __shared__ int flags[2];

    const int r = blockIdx.x;
    const int split = blockIdx.y;
    const int g = blockIdx.z;
    const int G = gridDim.z;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int b = row_seq[r];
    const bool row_ok = b >= 0 && b < B;
    const int s0 = split * split_len;
    const int s1 = min(s0 + split_len, W);

    // Query fragment for S^T = K Q^T (B operand): head column lane&15 of this wave's 16,
    // channels 32*st + (lane>>4)*8 .. +8 at step st.
    const int qk_head_local = 16 * (wave & 1) + (lane & 15);
    const int qk_head = g * 32 + qk_head_local;
    u32x4 qf[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) {
        qf[st] = u32x4{0u, 0u, 0u, 0u};
        if (qk_head < H)
            qf[st] = *reinterpret_cast<const u32x4 *>(q_abs + ((size_t)r * H + qk_head) * kC +
                                                      32 * st + (lane >> 4) * 8);
    }

    float m_run = -INFINITY;  // running max of head qk_head (same in waves w and w^2)
    float l_run = 0.0f;       // this lane's share of the running sum
    f32x16 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x16{};

    if (tid < 2) flags[tid] = 0;
    __syncthreads();

    const int tb = 16 * (wave >> 1);  // this wave's 16 tokens of the tile in S^T
    int it = 0;
    for (int t0 = s0; t0 < s1; t0 += kTile, ++it) {
        const int par = it & 1;
        // ---- gather: wave w stores tile rows 8w..8w+7; lane owns channels 8*lane..+8
        bool any = false;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row_in_tile = 8 * wave + j;
            const int slot = t0 + row_in_tile;
            const int tok = slot < s1 ? token_ids[(size_t)r * W + slot] : -1;
            long long row = -1;
            if (tok >= 0 && row_ok && (S <= 0 || tok < S)) {
                if constexpr (PAGED) {
                    const int blk = tok / block_size;
                    if (blk < max_blocks) {
                        const int pb = block_table[(size_t)b * max_blocks + blk];
                        if (pb >= 0) row = (long long)pb * block_size + (tok - blk * block_size);
                    }
                } else {
                    row = (long long)b * S + tok;
                }
                if (row >= kv_rows) row = -1;
            }
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row >= 0) {
                any = true;
                if constexpr (FP8) {
                    const u32x2 raw = *reinterpret_cast<const u32x2 *>(
                        static_cast<const uint8_t *>(kv) + row * kC + 8 * lane);
                    const u32x2 lo = e4m3x4_to_bf16x4(raw.x), hi = e4m3x4_to_bf16x4(raw.y);
                    x = u32x4{lo.x, lo.y, hi.x, hi.y};
                } else {
                    x = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(kv) +
                                                         row * kC + 8 * lane);
                }
            }
            *reinterpret_cast<u32x4 *>(kt + row_in_tile * kKtStride + 8 * lane) = x;
            if (lane == 0) {
                tok_ok[row_in_tile] = row >= 0;
                float sc = 1.0f;
                if constexpr (FP8) sc = row >= 0 ? kv_scales[row] : 0.0f;
                tok_scale[row_in_tile] = sc;
            }
        }
        if (any && lane == 0) flags[par] = 1;
        __syncthreads();  // A: tile, flags visible
        const bool live = flags[par] != 0;

        // ---- logits S^T[token][head] for this wave's 16 tokens x 16 heads
        float x[4];
        if (live) {
            f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(
                    kt + (tb + (lane & 15)) * kKtStride + 32 * st + (lane >> 4) * 8);
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qf[st]), s4,
                                                             0, 0, 0);
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tk = tb + (lane >> 4) * 4 + i;
                x[i] = tok_ok[tk] ? s4[i] * (sm_scale * tok_scale[tk]) : -INFINITY;
                tmax = fmaxf(tmax, x[i]);
            }
            tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
            tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
            if (lane < 16) red[wave][lane] = tmax;
        }
        __syncthreads();  // B: tile maxima
        if (live) {
            const float m_tile = fmaxf(red[wave][lane & 15], red[wave ^ 2][lane & 15]);
            const float m_new = fmaxf(m_run, m_tile);
            const float alpha = m_new == -INFINITY ? 1.0f : fast_exp(m_run - m_new);
            float psum = 0.0f;
            uint32_t pk[2];
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const int tk = tb + (lane >> 4) * 4 + i;
                const float p0 = x[i] == -INFINITY ? 0.0f : fast_exp(x[i] - m_new);
                const float p1 = x[i + 1] == -INFINITY ? 0.0f : fast_exp(x[i + 1] - m_new);
                psum += p0 + p1;
                pk[i >> 1] = pack_bf16x2(p0 * tok_scale[tk], p1 * tok_scale[tk + 1]);
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            *reinterpret_cast<u32x2 *>(pl + qk_head_local * kPStride + tb + (lane >> 4) * 4) =
                u32x2{pk[0], pk[1]};
            if ((wave >> 1) == 0 && lane < 16) alpha_s[qk_head_local] = alpha;
        }
        if (tid == 0) flags[par ^ 1] = 0;
        __syncthreads();  // C: P and alpha visible
        if (live) {
            // rescale: accumulator row (head) of register i is 8*(i/4) + 4*(lane>>5) + i%4
            float al[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) al[i] = alpha_s[8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[nt][i] *= al[i];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(pl + (lane & 31) * kPStride +
                                                                 16 * ks + (lane >> 5) * 8);
                const int tok0 = 16 * ks + (lane >> 5) * 8;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int ch = 128 * wave + 32 * nt + (lane & 31);
                    const uint16_t *col = kt + tok0 * kKtStride + ch;
                    u32x4 v;
                    v.x = (uint32_t)col[0] | ((uint32_t)col[kKtStride] << 16);
                    v.y = (uint32_t)col[2 * kKtStride] | ((uint32_t)col[3 * kKtStride] << 16);
                    v.z = (uint32_t)col[4 * kKtStride] | ((uint32_t)col[5 * kKtStride] << 16);
                    v.w = (uint32_t)col[6 * kKtStride] | ((uint32_t)col[7 * kKtStride] << 16);
                    acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(v),
                                                                      acc[nt], 0, 0, 0);
                }
            }
        }
        __syncthreads();  // D: tile consumed
    }

    // ---- finish: per-head sums (lanes sharing lane&15 within the wave, then the partner wave)
    l_run += shfl_xor_f(l_run, 16);
    l_run += shfl_xor_f(l_run, 32);
    if (lane < 16) red[wave][lane] = l_run;
    __syncthreads();
    if (wave < 2 && lane < 16) {
        lsum_s[qk_head_local] = red[wave][lane] + red[wave ^ 2][lane];
        msum_s[qk_head_local] = m_run;
    }
    __syncthreads();

    if (splits == 1) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int ch = 128 * wave + 32 * nt + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                const int hg = g * 32 + m;
                if (hg < H) {
                    const float L = lsum_s[m];
                    out[((size_t)r * H + hg) * kC + ch] = L > 0.0f ? acc[nt][i] / L : 0.0f;
                }
            }
        }
        if (lse != nullptr && tid < 32 && g * 32 + tid < H) {
            const float L = lsum_s[tid];
            lse[(size_t)r * H + g * 32 + tid] = L > 0.0f ? msum_s[tid] + logf(L) : -INFINITY;
        }
    } else {
        float *part = ws + (((size_t)r * G + g) * splits + split) * kPartFloats;
        if (tid < 32) {
            part[tid] = msum_s[tid];
            part[32 + tid] = lsum_s[tid];
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int ch = 128 * wave + 32 * nt + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                part[64 + m * kC + ch] = acc[nt][i];
            }
        }
    }
}

// Merge the per-split partial results of one (row, head group): log-sum-exp weights.
__global__ __launch_bounds__(kThreads) void mla_combine_kernel(int H, int splits,
                                                               const float *__restrict__ ws,
                                                               float *__restrict__ out,
                                                               float *__restrict__ lse) {
    const int r = blockIdx.x;
    const int g = blockIdx.y;
    const int G = gridDim.y;
    const int tid = threadIdx.x;
    const float *base = ws + ((size_t)r * G + g) * splits * kPartFloats;
    for (int m = 0; m < 32; ++m) {
        const int hg = g * 32 + m;
        if (hg >= H) break;
        float M = -INFINITY;
        for (int s = 0; s < splits; ++s) M = fmaxf(M, base[(size_t)s * kPartFloats + m]);
        float L = 0.0f;
        for (int s = 0; s < splits; ++s) {
            const float ms = base[(size_t)s * kPartFloats + m];
            if (ms != -INFINITY) L += base[(size_t)s * kPartFloats + 32 + m] * fast_exp(ms - M);
        }
        for (int c = tid; c < kC; c += kThreads) {
            float o = 0.0f;
            for (int s = 0; s < splits; ++s) {
                const float ms = base[(size_t)s * kPartFloats + m];
                if (ms != -INFINITY)
                    o += base[(size_t)s * kPartFloats + 64 + m * kC + c] * fast_exp(ms - M);
            }
            out[((size_t)r * H + hg) * kC + c] = L > 0.0f ? o / L : 0.0f;
        }
        if (lse != nullptr && tid == 0) lse[(size_t)r * H + hg] = L > 0.0f ? M + logf(L) : -INFINITY;
    }
}

template <bool FP8, bool PAGED>
hipError_t launch_v(const MlaPlan &plan, int Q, int W, int H, int B, float sm_scale,
                    const uint16_t *q_abs, const int32_t *token_ids, const int32_t *row_seq,
                    const void *kv, const float *kv_scales, int64_t kv_rows, int S,
                    const int32_t *block_table, int max_blocks, int block_size, float *out,
                    float *lse, void *ws, hipStream_t stream) {
    hipLaunchKernelGGL((sparse_mla_kernel<FP8, PAGED>), dim3(Q, plan.splits, plan.groups),
                       dim3(kThreads), 0, stream, W, H, B, plan.splits, plan.split_len, sm_scale,
                       q_abs, token_ids, row_seq, kv, kv_scales, (long long)kv_rows, S,
                       block_table, max_blocks, block_size, out, lse,
                       static_cast<float *>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    hipLaunchKernelGGL(mla_combine_kernel, dim3(Q, plan.groups), dim3(kThreads), 0, stream, H,
                       plan.splits, static_cast<const float *>(ws), out, lse);
    return hipGetLastError();
}

}  // namespace

// Split the token slots so that about 512 blocks (two per compute unit) are in flight,
// with at least 64 slots per split; a row that already gives enough blocks is not split.
MlaPlan plan_sparse_mla(int Q, int W, int H) {
    MlaPlan p;
    p.groups = (H + 31) / 32;
    const long long work = (long long)W * Q * p.groups;
    long long per = (work + 511) / 512;
    per = ((per + kTile - 1) / kTile) * kTile;
    if (per < 64) per = 64;
    const long long wr = ((long long)W + kTile - 1) / kTile * kTile;
    if (per > wr) per = wr;
    if (per < kTile) per = kTile;
    p.splits = W > 0 ? (int)((W + per - 1) / per) : 1;
    if (p.splits > 1) {
        per = ((W + p.splits - 1) / p.splits + kTile - 1) / kTile * kTile;
        p.splits = (int)((W + per - 1) / per);
    }
    p.split_len = (int)per;
    p.ws_bytes = p.splits > 1 ? (size_t)Q * p.groups * p.splits * kPartFloats * sizeof(float) : 0;
    return p;
}

hipError_t launch_sparse_mla(const MlaPlan &plan, int Q, int W, int H, int B, float sm_scale,
                             const uint16_t *q_abs, const int32_t *token_ids,
                             const int32_t *row_seq, const void *kv, bool kv_fp8,
                             const float *kv_scales, int64_t kv_rows, int S,
                             const int32_t *block_table, int max_blocks, int block_size,
                             float *out, float *lse, void *ws, hipStream_t stream) {
    if (Q == 0) return hipSuccess;
    const bool paged = block_table != nullptr;
    if (kv_fp8)
        return paged ? launch_v<true, true>(plan, Q, W, H, B, sm_scale, q_abs, token_ids, row_seq,
                                            kv, kv_scales, kv_rows, S, block_table, max_blocks,
                                            block_size, out, lse, ws, stream)
                     : launch_v<true, false>(plan, Q, W, H, B, sm_scale, q_abs, token_ids,
                                             row_seq, kv, kv_scales, kv_rows, S, block_table,
                                             max_blocks, block_size, out, lse, ws, stream);
    return paged ? launch_v<false, true>(plan, Q, W, H, B, sm_scale, q_abs, token_ids, row_seq, kv,
                                         kv_scales, kv_rows, S, block_table, max_blocks,
                                         block_size, out, lse, ws, stream)
                 : launch_v<false, false>(plan, Q, W, H, B, sm_scale, q_abs, token_ids, row_seq,
                                          kv, kv_scales, kv_rows, S, block_table, max_blocks,
                                          block_size, out, lse, ws, stream);
}

}  // namespace dsa

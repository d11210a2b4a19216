// index_scores.hip -- pooled-key indexer scores.
//
// tp.rs, "Why the indexer is replicated": score[r, p] = sum_h w[r, h] * relu(scale * q_h . k_p).
// build.rs transform 2: w already carries index_heads^-0.5.
//
// The scorer is a dense contraction [heads x D] x [D x pools] per query row, so it runs on
// MFMA: v_mfma_f32_32x32x16_bf16 with the (up to 32) indexer heads as M and 32 pools as N.
// The query fragment stays in registers for the whole block; each lane streams one half of
// one pooled-key row (D/2 channels: 64 contiguous bytes of bf16, or 32 of fp8 converted to
// bf16 exactly in registers). Because the dot product does not depend on the order of its
// terms, lane half h simply owns channels [h*D/2, (h+1)*D/2) in both operands. The head
// reduction is fused in the epilogue: each lane holds 16 heads of one pool column, applies
// relu and the head weight, and one cross-lane add with the partner lane (lane ^ 32) finishes
// the column. Only the [Q, P] score row ever reaches memory.
//
// Work split: block (c, r) takes compacted entries [c*256, c*256 + 256) of row r's sequence,
// 4 waves x 2 tiles of 32 pools. The block also owns the pool-id range from just after the
// previous block's last id up to its own last id (through P for the last active block) and
// writes -inf / cand 0 over the non-candidate ids in it, so every slot of the score row is
// written exactly once and no fill pass is needed.
//
// Bytes per candidate pool: D*2 (bf16 key) or D + 4 (fp8 key and scale), plus 4 (id); the
// score row costs 5 bytes per pool slot.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kTilesPerWave = 2;
constexpr int kChunk = (kThreads / kWave) * kTilesPerWave * 32;

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void index_scores_kernel(
    int B, int P, int Hi, int KP, int first_key, float scale, const uint16_t *__restrict__ q,
    const float *__restrict__ w, const int32_t *__restrict__ row_seq,
    const int32_t *__restrict__ row_pos, const void *__restrict__ keys,
    const float *__restrict__ key_scales, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ n_valid, float *__restrict__ scores, uint8_t *__restrict__ cand) {
    constexpr int kSteps = D / 16;  // MFMA K-steps of 16 channels (8 per lane half)
    constexpr int kHalf = D / 2;
    __shared__ __attribute__((aligned(16))) uint16_t q_s[32 * D];
    __shared__ float w_s[32];

    const int r = blockIdx.y;
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    float *srow = scores + (size_t)r * P;
    uint8_t *crow = cand + (size_t)r * P;

    const int b = row_seq[r];
    const bool row_ok = b >= 0 && b < B;
    const long long pos = row_pos[r];
    int nv = row_ok ? n_valid[b] : 0;
    nv = nv < 0 ? 0 : (nv > P ? P : nv);
    const int j0 = c * kChunk;
    if (c != 0 && j0 >= nv) return;
    const int j1 = min(j0 + kChunk, nv);
    const int32_t *idrow = ids + (size_t)(row_ok ? b : 0) * P;
    auto clampP = [P](int v) { return v < 0 ? 0 : (v > P ? P : v); };
    const int lo = j0 == 0 ? 0 : clampP(idrow[j0 - 1] + 1);
    const int hi = j1 >= nv ? P : clampP(idrow[j1 - 1] + 1);

    // Non-candidate ids inside the owned range: the gap before each listed id ...
    for (int j = j0 + tid; j < j1; j += kThreads) {
        const int prev = j == j0 ? lo : clampP(idrow[j - 1] + 1);
        const int cur = min(clampP(idrow[j]), hi);
        for (int p = prev; p < cur; ++p) {
            srow[p] = -INFINITY;
            crow[p] = 0;
        }
    }
    // ... and the gap after the last one.
    {
        const int start = j1 > j0 ? clampP(idrow[j1 - 1] + 1) : lo;
        for (int p = start + tid; p < hi; p += kThreads) {
            srow[p] = -INFINITY;
            crow[p] = 0;
        }
    }
    if (j1 <= j0) return;

    // Stage the row's query (heads padded to 32 with zeros) and head weights.
    for (int e = tid * 8; e < 32 * D; e += kThreads * 8) {
        const int h = e / D;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < Hi) v = *reinterpret_cast<const u32x4 *>(q + ((size_t)r * Hi) * D + e);
        *reinterpret_cast<u32x4 *>(q_s + e) = v;
    }
    if (tid < 32) w_s[tid] = tid < Hi ? w[(size_t)r * Hi + tid] : 0.0f;
    __syncthreads();

    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n = lane & 31;
    const int half = lane >> 5;

    u32x4 qa[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
        qa[s] = *reinterpret_cast<const u32x4 *>(q_s + n * D + half * kHalf + s * 8);
    float wr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) wr[i] = w_s[8 * (i >> 2) + 4 * half + (i & 3)];

    for (int t = 0; t < kTilesPerWave; ++t) {
        const int jt = j0 + (t * (kThreads / kWave) + wave) * 32;
        if (jt >= j1) break;
        const int j = jt + n;
        int p = j < j1 ? idrow[j] : -1;
        const bool have = p >= 0 && p < P;
        if (!have) p = 0;
        const bool is_cand = have && (long long)first_key + (long long)(p + 1) * KP - 1 <= pos;

        // Every lane loads a real key row (p is in range), so no load is predicated; a column
        // that is not a candidate is dropped in the epilogue, and MFMA columns never mix.
        u32x4 kb[kSteps];
        if constexpr (FP8) {
            const uint8_t *krow =
                static_cast<const uint8_t *>(keys) + ((size_t)b * P + p) * D + half * kHalf;
#pragma unroll
            for (int ch = 0; ch < kHalf / 16; ++ch) {
                const u32x4 raw = *reinterpret_cast<const u32x4 *>(krow + ch * 16);
                const u32x2 a = e4m3x4_to_bf16x4(raw.x), bb = e4m3x4_to_bf16x4(raw.y);
                const u32x2 cc = e4m3x4_to_bf16x4(raw.z), d = e4m3x4_to_bf16x4(raw.w);
                kb[2 * ch] = u32x4{a.x, a.y, bb.x, bb.y};
                kb[2 * ch + 1] = u32x4{cc.x, cc.y, d.x, d.y};
            }
        } else {
            const uint16_t *krow =
                static_cast<const uint16_t *>(keys) + ((size_t)b * P + p) * D + half * kHalf;
#pragma unroll
            for (int s = 0; s < kSteps; ++s) kb[s] = *reinterpret_cast<const u32x4 *>(krow + s * 8);
        }
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[s]), as_bf16x8(kb[s]), acc,
                                                          0, 0, 0);
        float f = scale;
        if constexpr (FP8) f *= key_scales[(size_t)b * P + p];
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) part += wr[i] * fmaxf(acc[i] * f, 0.0f);
        float tot = part + shfl_xor_f(part, 32);
        if (tot == 0.0f) tot = 0.0f;
        if (half == 0 && have) {
            srow[p] = is_cand ? tot : -INFINITY;
            crow[p] = is_cand ? 1 : 0;
        }
    }
}

template <int D, bool FP8>
hipError_t launch_d(int Q, int B, int P, int Hi, int KP, int first_key, float scale,
                    const uint16_t *q, const float *w, const int32_t *row_seq,
                    const int32_t *row_pos, const void *keys, const float *key_scales,
                    const int32_t *ids, const int32_t *n_valid, float *scores, uint8_t *cand,
                    hipStream_t stream) {
    const int chunks = P > 0 ? (P + kChunk - 1) / kChunk : 1;
    hipLaunchKernelGGL((index_scores_kernel<D, FP8>), dim3(chunks, Q), dim3(kThreads), 0, stream,
                       B, P, Hi, KP, first_key, scale, q, w, row_seq, row_pos, keys, key_scales,
                       ids, n_valid, scores, cand);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores(int Q, int B, int P, int Hi, int D, int KP, int first_key,
                               float scale, const uint16_t *q, const float *w,
                               const int32_t *row_seq, const int32_t *row_pos, const void *keys,
                               bool key_fp8, const float *key_scales, const int32_t *ids,
                               const int32_t *n_valid, float *scores, uint8_t *cand,
                               hipStream_t stream) {
    if (Q == 0 || P == 0) return hipSuccess;
#define DSA_IS_CASE(d)                                                                       \
    if (D == d)                                                                              \
        return key_fp8 ? launch_d<d, true>(Q, B, P, Hi, KP, first_key, scale, q, w, row_seq, \
                                           row_pos, keys, key_scales, ids, n_valid, scores,  \
                                           cand, stream)                                     \
                       : launch_d<d, false>(Q, B, P, Hi, KP, first_key, scale, q, w, row_seq, \
                                            row_pos, keys, key_scales, ids, n_valid, scores, \
                                            cand, stream);
    DSA_IS_CASE(32)
    DSA_IS_CASE(64)
    DSA_IS_CASE(128)
#undef DSA_IS_CASE
    return hipErrorInvalidValue;
}

}  // namespace dsa

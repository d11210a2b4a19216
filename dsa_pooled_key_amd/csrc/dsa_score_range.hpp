// dsa_score_range.hpp -- the pool scores of one block's slot range (compaction and scoring
// of one row, from the validity flags).
//
// tp.rs, "Why the indexer is replicated": score[r, p] = sum_h w[r, h] * relu(scale * q_h . k_p),
// build.rs transform 2 (w carries index_heads^-0.5); mod.rs, "Shape of the pipeline": only
// valid pools are scored (the compaction step). A block of NT threads takes slots
// [slot0, slot0 + NT/64 * TPW * 32) of row r: wave w's tile t is slots slot0 + (t*NT/64 + w)*32
// .. +31, lane n (and its partner n + 32, which holds the other half of the channels) owning
// slot n of the tile. The flags of those slots are read once the row's sequence is known, and a
// pooled key is requested only for a slot that is valid and whose last token is at or before the
// row position, so the keys of invalid pools are never read (the saving a compacted id list
// exists for) and no id list is written or read. Every slot of the range is written by its lane:
// the score and cand = 1 for a candidate, -inf and cand = 0 otherwise. Two dependent round
// trips once the row's sequence and position are known: the query with the flags; the keys.
// Dot products run on v_mfma_f32_32x32x16_bf16 (heads as M, 32 pools as N); fp8 keys are
// converted to bf16 exactly in registers; the relu-weighted head sum is the epilogue.
#pragma once

#include "dsa_device.hpp"
#include "dsa_phase.hpp"

namespace dsa {

// LDS position (in bf16 elements) of the 16-byte chunk c of query head h: the chunks of each
// head row are XOR-rotated by the head index, so the 16 lanes of one ds_read_b128 pass (heads
// n..n+15, one chunk each) fall in distinct banks instead of all at the same offset of rows
// D*2 bytes apart.
template <int D>
__device__ __forceinline__ int q_slot(int h, int c) {
    return h * D + 8 * (c ^ (h & (D / 8 - 1)));
}

// Pools [0, limit) of a row at position pos end at or before it (and exist); 0 for a row whose
// sequence index is outside the batch.
__device__ __forceinline__ long long row_pool_limit(int b, long long pos, int B, int P, int KP,
                                                    int first_key) {
    if (b < 0 || b >= B) return 0;
    long long lim = pos + 1 > first_key ? (pos + 1 - first_key) / KP : 0;
    return lim > P ? P : lim;
}

// One lane's share of a pool's score: sum_i w_i * relu(f * acc_i) = f * sum_i w_i * clamp(acc_i),
// clamp = max(., 0) for f >= 0 and min(., 0) for f < 0 (one v_med3 against 0 and +-inf), so the
// scale multiplies once per pool instead of once per head.
__device__ __forceinline__ float relu_weighted(const f32x16 &acc, const float (&wr)[16], float f) {
    const float bound = f >= 0.0f ? INFINITY : -INFINITY;
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) part += wr[i] * __builtin_amdgcn_fmed3f(acc[i], 0.0f, bound);
    return part;
}

// b, pos: row r's sequence and position. q_s: LDS of 32*D bf16 (16-byte aligned); w_s: LDS of
// 32 floats. Ends with the block's stores issued (not waited for).
template <int D, bool FP8, int TPW, int NT>
__device__ __forceinline__ void score_range(
    int r, int b, long long pos, int slot0, int B, int P, int Hi, int KP, int first_key, float scale,
    const uint16_t *__restrict__ q, const float *__restrict__ w, const void *__restrict__ keys,
    const float *__restrict__ key_scales, const uint8_t *__restrict__ pool_valid,
    float *__restrict__ scores, uint8_t *__restrict__ cand, uint16_t *q_s, float *w_s) {
    constexpr int kSteps = D / 16;
    constexpr int kHalf = D / 2;
    constexpr int kQVec = 32 * D / 8;
    constexpr int kWaves = NT / kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n = lane & 31;
    const int half = lane >> 5;
    float *srow = scores + (size_t)r * P;
    uint8_t *crow = cand + (size_t)r * P;

    // Round trip 1: the row's query and head weights (its sequence b and position pos are
    // the caller's), and with them the flags below.
    u32x4 qv[(kQVec + NT - 1) / NT];
#pragma unroll
    for (int k = 0; k < (kQVec + NT - 1) / NT; ++k) {
        const int e = (tid + k * NT) * 8;
        const int h = e / D;
        qv[k] = u32x4{0u, 0u, 0u, 0u};
        if (e < 32 * D && h < Hi) qv[k] = *reinterpret_cast<const u32x4 *>(q + ((size_t)r * Hi) * D + e);
    }
    const float wv = tid < 32 && tid < Hi ? w[(size_t)r * Hi + tid] : 0.0f;
    const long long lim = row_pool_limit(b, pos, B, P, KP, first_key);

    DSA_PHASE(0, 1);  // range known, query requested
    // The validity flags of this lane's slots, then (round trip 2) their keys. The
    // flags sit under one branch that is uniform over the wave (a lane past the row's limit
    // reads the last flag in range and drops it), so they are requested together: under a
    // branch per tile the compiler waits for each flag before requesting the next.
    int slot[TPW];
    bool ok[TPW];
    uint32_t flag[TPW];
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        slot[t] = slot0 + (t * kWaves + wave) * 32 + n;
        flag[t] = 0u;
    }
    if (slot0 + wave_u * 32 < lim) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            flag[t] = pool_valid[(size_t)b * P + (slot[t] < lim ? slot[t] : (int)lim - 1)];
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) ok[t] = slot[t] < lim && flag[t] != 0u;
    u32x4 raw[TPW][FP8 ? kHalf / 16 : kSteps];
    float ksc[TPW];
    bool any[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        // The wave skips a tile with no candidate; otherwise a lane without one fetches nothing
        // and its column is dropped.
        any[t] = __builtin_amdgcn_ballot_w64(ok[t]) != 0;
        ksc[t] = 1.0f;
#pragma unroll
        for (int k = 0; k < (FP8 ? kHalf / 16 : kSteps); ++k) raw[t][k] = u32x4{0u, 0u, 0u, 0u};
        if (ok[t]) {
            const size_t kr = (size_t)b * P + slot[t];
            if constexpr (FP8) {
                const uint8_t *krow = static_cast<const uint8_t *>(keys) + kr * D + half * kHalf;
#pragma unroll
                for (int ch = 0; ch < kHalf / 16; ++ch) raw[t][ch] = *reinterpret_cast<const u32x4 *>(krow + ch * 16);
                ksc[t] = key_scales[kr];
            } else {
                const uint16_t *krow = static_cast<const uint16_t *>(keys) + kr * D + half * kHalf;
#pragma unroll
                for (int st = 0; st < kSteps; ++st) raw[t][st] = *reinterpret_cast<const u32x4 *>(krow + st * 8);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < (kQVec + NT - 1) / NT; ++k) {
        const int e = (tid + k * NT) * 8;
        if (e < 32 * D) *reinterpret_cast<u32x4 *>(q_s + q_slot<D>(e / D, (e % D) / 8)) = qv[k];
    }
    if (tid < 32) w_s[tid] = wv;
    __syncthreads();
    DSA_PHASE(0, 2);  // query and flags landed, query staged

    float wr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) wr[i] = w_s[8 * (i >> 2) + 4 * half + (i & 3)];

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        float tot = 0.0f;
        if (any[t]) {
            f32x16 acc = {};
#pragma unroll
            for (int st = 0; st < kSteps; ++st) {
                u32x4 kb;
                if constexpr (FP8) {
                    const u32x4 rw = raw[t][st >> 1];
                    kb = (st & 1) ? e4m3x8_to_bf16x8(rw.z, rw.w) : e4m3x8_to_bf16x8(rw.x, rw.y);
                } else {
                    kb = raw[t][st];
                }
                const u32x4 qa = *reinterpret_cast<const u32x4 *>(q_s + q_slot<D>(n, half * (kHalf / 8) + st));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa), as_bf16x8(kb), acc, 0, 0, 0);
            }
            const float f = scale * ksc[t];
            tot = f * add_xor32(relu_weighted(acc, wr, f));
            if (t == 0) DSA_PHASE(0, 3);  // keys landed, first tile scored
            if (tot == 0.0f) tot = 0.0f;
        }
        if (half == 0 && slot[t] < P) {
            srow[slot[t]] = ok[t] ? tot : -INFINITY;
            crow[slot[t]] = ok[t] ? 1 : 0;
        }
    }
}

}  // namespace dsa

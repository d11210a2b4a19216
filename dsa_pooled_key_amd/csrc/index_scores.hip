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
// Work split: block (r, c) takes compacted entries [c*256, c*256 + 256) of row r's sequence,
// 4 waves x 2 tiles of 32 pools, in three dependent round trips (row geometry and query; the
// count and the block's ids; the keys). The block writes -inf / cand 0 over the ids that are
// not listed between the previous block's last id and its own last id, and over the ids past
// the end of the list that fall in its stripe [c*256, c*256 + 256); so every slot of the score
// row is written exactly once and no fill pass is needed.
//
// Bytes per candidate pool: D*2 (bf16 key) or D + 4 (fp8 key and scale), plus 4 (id); the
// score row costs 5 bytes per pool slot.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <mutex>

#include "dsa_device.hpp"
#include "dsa_launch.hpp"
#include "dsa_phase.hpp"

DSA_PHASE_TABLE(scores)

#include "dsa_score_range.hpp"

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
    constexpr int kQVec = 32 * D / 8;  // 16-byte pieces of the padded query block
    __shared__ __attribute__((aligned(16))) uint16_t q_s[32 * D];
    __shared__ float w_s[32];
    __shared__ int ids_s[kChunk + 1];  // ids[j0 - 1 .. j0 + kChunk - 1]

    const int r = blockIdx.x;  // rows vary fastest, so every row's first chunks (the ones
    const int c = blockIdx.y;  // that hold entries) are dispatched before the empty ones
    const int tid = threadIdx.x;
    float *srow = scores + (size_t)r * P;
    uint8_t *crow = cand + (size_t)r * P;
    const int j0 = c * kChunk;

    // Round trip 1: everything that does not depend on the row's sequence.
    const int b = row_seq[r];
    const long long pos = row_pos[r];
    u32x4 qv[(kQVec + kThreads - 1) / kThreads];
#pragma unroll
    for (int k = 0; k < (kQVec + kThreads - 1) / kThreads; ++k) {
        const int e = (tid + k * kThreads) * 8;  // first element of this piece
        const int h = e / D;
        qv[k] = u32x4{0u, 0u, 0u, 0u};
        if (e < 32 * D && h < Hi) qv[k] = *reinterpret_cast<const u32x4 *>(q + ((size_t)r * Hi) * D + e);
    }
    const float wv = tid < 32 && tid < Hi ? w[(size_t)r * Hi + tid] : 0.0f;
    // Round trip 2: the sequence's valid count and this block's slice of its id list.
    const bool row_ok = b >= 0 && b < B;
    int nv = row_ok ? n_valid[b] : 0;
    nv = nv < 0 ? 0 : (nv > P ? P : nv);
    const int32_t *idrow = ids + (size_t)(row_ok ? b : 0) * P;
    const int my_id = j0 + tid < P ? idrow[j0 + tid] : -1;
    const int prev_id = (tid == 0 && j0 > 0) ? idrow[j0 - 1] : -1;
#pragma unroll
    for (int k = 0; k < (kQVec + kThreads - 1) / kThreads; ++k) {
        const int e = (tid + k * kThreads) * 8;
        if (e < 32 * D) *reinterpret_cast<u32x4 *>(q_s + q_slot<D>(e / D, (e % D) / 8)) = qv[k];
    }
    if (tid < 32) w_s[tid] = wv;
    ids_s[1 + tid] = my_id;
    if (tid == 0) ids_s[0] = prev_id;
    __syncthreads();
    const int j1 = min(j0 + kChunk, nv);
    auto clampP = [P](int v) { return v < 0 ? 0 : (v > P ? P : v); };
    auto id_at = [&](int j) { return ids_s[j - j0 + 1]; };  // j in [j0 - 1, j0 + kChunk)
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n = lane & 31;
    const int half = lane >> 5;

    // Round trip 3: both tiles' pooled-key half rows are requested before any product, and
    // with them the id that ends the list (the pools after it are written in stripes below).
    int pt[kTilesPerWave];
    bool have[kTilesPerWave], active[kTilesPerWave];
    u32x4 raw[kTilesPerWave][FP8 ? kHalf / 16 : kSteps];
    float ksc[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
        const int jt = j0 + (t * (kThreads / kWave) + wave) * 32;
        active[t] = jt < j1;
        const int j = jt + n;
        int p = (active[t] && j < j1) ? id_at(j) : -1;
        have[t] = p >= 0 && p < P;
        if (!have[t]) p = 0;  // a real row: no load is predicated; the column is dropped later
        pt[t] = p;
        ksc[t] = 1.0f;
        if (active[t]) {
            if constexpr (FP8) {
                const uint8_t *krow =
                    static_cast<const uint8_t *>(keys) + ((size_t)b * P + p) * D + half * kHalf;
#pragma unroll
                for (int ch = 0; ch < kHalf / 16; ++ch) raw[t][ch] = *reinterpret_cast<const u32x4 *>(krow + ch * 16);
                ksc[t] = key_scales[(size_t)b * P + p];
            } else {
                const uint16_t *krow =
                    static_cast<const uint16_t *>(keys) + ((size_t)b * P + p) * D + half * kHalf;
#pragma unroll
                for (int s = 0; s < kSteps; ++s) raw[t][s] = *reinterpret_cast<const u32x4 *>(krow + s * 8);
            }
        }
    }
    const int tail = nv > 0 ? clampP(idrow[nv - 1] + 1) : 0;  // first pool after the last listed id

    // Every slot of the score row is written once. Non-candidate ids between this block's
    // listed ids: the gap before each of them (from just after the previous block's last id)
    // ...
    if (j1 > j0) {
        const int lo = j0 == 0 ? 0 : clampP(id_at(j0 - 1) + 1);
        for (int j = j0 + tid; j < j1; j += kThreads) {
            const int prev = j == j0 ? lo : clampP(id_at(j - 1) + 1);
            const int cur = clampP(id_at(j));
            for (int p = prev; p < cur; ++p) {
                srow[p] = -INFINITY;
                crow[p] = 0;
            }
        }
    }
    // ... and, in stripes of kChunk pool ids (block c takes [c*kChunk, c*kChunk + kChunk)), every
    // pool after the last listed id (written at the end, once that id has arrived).
    auto fill_tail = [&]() {
        const int p = j0 + tid;
        if (p >= tail && p < P) {
            srow[p] = -INFINITY;
            crow[p] = 0;
        }
    };
    if (j1 <= j0) {
        fill_tail();
        return;
    }

    // The query fragment (A operand: head n, channels half*D/2 + 8s ..) is read from LDS at
    // each step (swizzled, conflict-free), which leaves registers for both tiles' keys.
    float wr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) wr[i] = w_s[8 * (i >> 2) + 4 * half + (i & 3)];

#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
        if (!active[t]) break;
        const int p = pt[t];
        const bool is_cand = have[t] && (long long)first_key + (long long)(p + 1) * KP - 1 <= pos;
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4 kb;
            if constexpr (FP8) {
                const u32x4 rw = raw[t][s >> 1];
                kb = (s & 1) ? e4m3x8_to_bf16x8(rw.z, rw.w) : e4m3x8_to_bf16x8(rw.x, rw.y);
            } else {
                kb = raw[t][s];
            }
            const u32x4 qa = *reinterpret_cast<const u32x4 *>(q_s + q_slot<D>(n, half * (kHalf / 8) + s));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa), as_bf16x8(kb), acc, 0, 0, 0);
        }
        const float f = scale * ksc[t];
        float tot = f * add_xor32(relu_weighted(acc, wr, f));
        if (tot == 0.0f) tot = 0.0f;
        if (half == 0 && have[t]) {
            srow[p] = is_cand ? tot : -INFINITY;
            crow[p] = is_cand ? 1 : 0;
        }
    }
    fill_tail();
}

// The compaction and the scoring in one launch: each (row, chunk) range of pool slots is scored
// by score_range. With up to kThreads rows, the ranges are ordered so that those holding
// candidates come first, row after row, and the ranges past a row's limit after them; the
// order costs one block scan over the rows' positions. Block j takes range j of that order
// (consecutive blocks land on different CUs, so a long row's ranges spread over the chip).
// When the ranges outnumber the blocks resident at once (WALK), the grid holds only that many
// blocks and each walks its ranges: with fewer ranges holding candidates (A) than blocks, block
// j < A takes the j-th such range and the idle ranges, which need only their -inf fill, are
// dealt to the remaining blocks, so none starts behind a scoring block; otherwise every block
// takes the ranges j, j + N, ... of the whole order. (A separate instantiation: the walk costs
// registers, which the one-range form keeps for occupancy.) Without the order (more rows than
// threads), range L is (row L % Q, chunk L / Q).
template <int D, bool FP8, int TPW, bool WALK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void index_scores_valid_kernel(
    int Q, int chunks, int B, int P, int Hi, int KP, int first_key, float scale,
    const uint16_t *__restrict__ q, const float *__restrict__ w, const int32_t *__restrict__ row_seq,
    const int32_t *__restrict__ row_pos, const void *__restrict__ keys,
    const float *__restrict__ key_scales, const uint8_t *__restrict__ pool_valid,
    float *__restrict__ scores, uint8_t *__restrict__ cand) {
    constexpr int kChunkV = (kThreads / kWave) * TPW * 32;
    __shared__ __attribute__((aligned(16))) uint16_t q_s[32 * D];
    __shared__ float w_s[32];
    __shared__ int scan_s[kThreads / kWave + 1];
    __shared__ int item_s[2];
    __shared__ int seq_s[kThreads];
    __shared__ long long pos_s[kThreads];
    DSA_PHASE(0, 0);  // block start
    const int total = Q * chunks;
    const int N = gridDim.x;
    const int j = blockIdx.x;
    const int t = threadIdx.x;
    // Range L of the block's walk: its row and chunk, with the row's geometry.
    auto run = [&](int r, int c, int b, long long pos) {
        const long long lim = row_pool_limit(b, pos, B, P, KP, first_key);
        const int slot0 = c * kChunkV;
        if (slot0 >= lim) {  // no candidate in the range (uniform over the block): the fill only
            for (int s = slot0 + t; s < min(slot0 + kChunkV, P); s += kThreads) {
                scores[(size_t)r * P + s] = -INFINITY;
                cand[(size_t)r * P + s] = 0;
            }
            return;
        }
        score_range<D, FP8, TPW, kThreads>(r, b, pos, slot0, B, P, Hi, KP, first_key, scale, q, w,
                                           keys, key_scales, pool_valid, scores, cand, q_s, w_s);
        DSA_PHASE(0, 4);  // range scored, stores issued
    };
    if (Q <= kThreads && total < (1 << 15)) {
        int act = 0;  // ranges of row t holding candidates
        if (t < Q) {
            const int bt = row_seq[t];
            const long long pt = row_pos[t];
            seq_s[t] = bt;  // every row's geometry stays in LDS for the block's ranges
            pos_s[t] = pt;
            const long long lim = row_pool_limit(bt, pt, B, P, KP, first_key);
            act = (int)((lim + kChunkV - 1) / kChunkV);
        }
        const int idle = t < Q ? chunks - act : 0;
        int tot;  // both counts in one scan (each sum is below Q * chunks < 2^15)
        const int pre = block_exclusive_scan<kThreads>(act | (idle << 15), scan_s, &tot);
        const int pa = pre & 0x7fff, pi = pre >> 15, A = tot & 0x7fff;
        // Range L of the order: its row and chunk (the row's thread publishes them).
        auto find = [&](int L) {
            if (t < Q) {
                if (L < A) {
                    if (L >= pa && L < pa + act) item_s[0] = t, item_s[1] = L - pa;
                } else if (L - A >= pi && L - A < pi + idle) {
                    item_s[0] = t, item_s[1] = act + (L - A - pi);
                }
            }
            __syncthreads();
        };
        if constexpr (!WALK) {
            find(j);
            const int r = min(max(item_s[0], 0), Q - 1);
            const int c = min(max(item_s[1], 0), chunks - 1);
            run(r, c, seq_s[r], pos_s[r]);
        } else {
            // The block's ranges: L0, L0 + step, ... below total.
            int L0 = j, step = N;
            const int idle_blocks = N - A, idle_ranges = total - A;
            if (A < N && idle_ranges <= 4 * idle_blocks) {
                if (j < A) step = total;  // its one range with candidates
                else L0 = A + (j - A), step = idle_blocks;
            }
            for (int L = L0; L < total; L += step) {
                if (L != L0) __syncthreads();  // the previous range is done with q_s, w_s and item_s
                find(L);
                const int r = min(max(item_s[0], 0), Q - 1);
                const int c = min(max(item_s[1], 0), chunks - 1);
                run(r, c, seq_s[r], pos_s[r]);
            }
        }
    } else if constexpr (!WALK) {
        run(j % Q, j / Q, row_seq[j % Q], row_pos[j % Q]);
    } else {
        for (int L = j; L < total; L += N) {
            if (L != j) __syncthreads();  // the previous range is done with q_s and w_s
            const int r = L % Q;
            run(r, L / Q, row_seq[r], row_pos[r]);
        }
    }
}

// Rows that all read one sequence's keys (prefill: consecutive positions of one sequence), as
// a blocked product: block (g, c) scores rows 16g..16g+15 against pools [2048c, 2048c + 2048)
// in sixteen tiles of 128 pools. A tile's keys are copied HBM->LDS (global_load_lds_dwordx4,
// each pool row's 16-byte chunks XOR-rotated by the pool index so the 16 lanes of a fragment
// read fall in distinct banks) into one of two buffers while the other is multiplied, and
// reused by all 16 rows (eight waves; with 8 rows and four waves a block the scorer took 290
// against 283 us on prefill_2048_64k, the copies being twice as many); wave w keeps the query
// fragments of rows 16g+2w and 16g+2w+1 in registers for the whole block and runs, per 32-pool
// sub-tile, the two rows' 32-head x 32-pool products on v_mfma_f32_32x32x16_bf16 from the same
// key fragments. Candidacy (the pool's flag and the
// row's causal limit) and the relu-weighted head sum are the epilogue, as in the per-row form;
// a tile's results are stored at the start of the next iteration, ahead of that iteration's
// copies, so the wait that ends it finds them done.
constexpr int kRB = 16;     // rows a block
constexpr int kRBThreads = kRB * 32;  // two rows a wave
constexpr int kCB = 128;    // pools a key tile
constexpr int kTiles = 16;  // key tiles a block

template <int D, bool FP8>
__global__ __launch_bounds__(kRBThreads) __attribute__((amdgpu_waves_per_eu(2))) void index_scores_rowblock_kernel(
    int Q, int P, int Hi, int KP, int first_key, float scale, const uint16_t *__restrict__ q,
    const float *__restrict__ w, const int32_t *__restrict__ row_seq,
    const int32_t *__restrict__ row_pos, const void *__restrict__ keys,
    const float *__restrict__ key_scales, const uint8_t *__restrict__ pool_valid,
    float *__restrict__ scores, uint8_t *__restrict__ cand) {
    constexpr int kSteps = D / 16;
    constexpr int kRowBytes = FP8 ? D : 2 * D;       // one pool's key row
    constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks a key row
    constexpr int kTileBytes = kCB * kRowBytes;
    constexpr int kCopies = kTileBytes / 1024;       // wave-wide 1 KiB copies a tile
    constexpr int kCopiesPerWave = (kCopies + kRBThreads / kWave - 1) / (kRBThreads / kWave);
    static_assert(kCopiesPerWave >= 1, "tile copies");
    constexpr int kSub = kCB / 32;                   // 32-pool sub-tiles a tile
    __shared__ __attribute__((aligned(16))) uint8_t ktile[2][kTileBytes];
    __shared__ __attribute__((aligned(16))) float ks_s[2][kCB];
    __shared__ float w_s[kRB][32];
    __shared__ int lim_s[kRB];
    __shared__ __attribute__((aligned(16))) uint8_t fl_s[kCB * kTiles];

    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n = lane & 31;
    const int half = lane >> 5;
    const int pbase = blockIdx.y * kCB * kTiles;
    const int ntiles = min(kTiles, (P - pbase + kCB - 1) / kCB);
    const uint8_t *kb8 = static_cast<const uint8_t *>(keys);
    auto kpos = [&](int p, int ch) { return p * kRowBytes + 16 * (ch ^ (p & (kChunks - 1))); };

    // Copy of tile it into buffer it&1: copy d of the tile lands at byte 1024d, lane l's 16
    // bytes at pool row (1024d + 16l) / kRowBytes, chunk position j; the lane fetches the
    // source chunk that belongs at j. Pools past P read pool P-1 (never used).
    auto issue_tile = [&](int it) {
        const int p0 = pbase + it * kCB;
#pragma unroll
        for (int k = 0; k < kCopiesPerWave; ++k) {
            const int d = wave * kCopiesPerWave + k;
            if (d >= kCopies) break;  // uniform over the wave
            const int p = (1024 * d + 16 * lane) / kRowBytes;
            const int j = lane % kChunks;
            const int pg = min(p0 + p, P - 1);
            dma16(kb8 + (size_t)pg * kRowBytes + 16 * (j ^ (p & (kChunks - 1))),
                  __builtin_amdgcn_readfirstlane(lds_offset(&ktile[it & 1][1024 * d])));
        }
        if constexpr (FP8) {
            if (wave < kCB / kWave)
                dma4(key_scales + min(p0 + kWave * wave + lane, P - 1),
                     __builtin_amdgcn_readfirstlane(lds_offset(&ks_s[it & 1][kWave * wave])));
        }
    };
    // Flags of this lane's pools of tile it (sub-tile t: pool 32t + n), as a bit mask, from the
    // block's flags in LDS.
    auto load_flags = [&](int it) {
        uint32_t m = 0u;
#pragma unroll
        for (int t = 0; t < kSub; ++t) m |= fl_s[it * kCB + 32 * t + n] != 0 ? 1u << t : 0u;
        return m;
    };

    // Prologue, one round trip: tile 0, its flags, the two rows' query fragments, the rows'
    // weights and limits (a row outside [0, Q) or of no sequence of the batch has none).
    issue_tile(0);
    // The block's flags (flags past P read as 0).
    for (int i = tid; i < kCB * kTiles; i += kRBThreads) fl_s[i] = pbase + i < P ? pool_valid[pbase + i] : 0;
    if (tid < kRB * 32) {
        const int rl = tid / 32, h = tid % 32, r = g * kRB + rl;
        w_s[rl][h] = r < Q && h < Hi ? w[(size_t)r * Hi + h] : 0.0f;
        if (h == 0)
            lim_s[rl] = r < Q ? (int)row_pool_limit(row_seq[r], row_pos[r], 1, P, KP, first_key) : 0;
    }
    const int r0 = g * kRB + 2 * wave;
    u32x4 qa[2][kSteps];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = min(r0 + j, Q - 1);
        const u32x4 *qrow = reinterpret_cast<const u32x4 *>(
            q + ((size_t)r * Hi + min(n, Hi - 1)) * D + half * (D / 2));
#pragma unroll
        for (int st = 0; st < kSteps; ++st) qa[j][st] = qrow[st];
    }
    wait_vm<0>();
    __syncthreads();
    uint32_t fl_next = load_flags(0);
    if (n >= Hi) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int st = 0; st < kSteps; ++st) qa[j][st] = u32x4{0u, 0u, 0u, 0u};
    }
    const int lim0 = lim_s[2 * wave], lim1 = lim_s[2 * wave + 1];
    float wr0[16], wr1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int h = 8 * (i >> 2) + 4 * half + (i & 3);
        wr0[i] = w_s[2 * wave][h];
        wr1[i] = w_s[2 * wave + 1][h];
    }

    // LDS offsets of this lane's key fragments within a 32-pool sub-tile (pool n): the chunk
    // rotation depends on the pool index only through n, so they are the same for every
    // sub-tile and buffer.
    constexpr int kFrags = FP8 ? kSteps / 2 : kSteps;
    uint32_t koff[kFrags];
#pragma unroll
    for (int k = 0; k < kFrags; ++k)
        koff[k] = (uint32_t)kpos(n, half * (FP8 ? D / 32 : D / 16) + k);

    // The previous tile's scores, stored at the next iteration's start: lane half h writes row
    // r0 + h (both halves hold both rows' sums).
    float res[kSub];
    uint32_t res_ok = 0u;
    int res_tile = -1;
    auto store_results = [&]() {
        const int r = r0 + half;
        if (res_tile < 0 || r >= Q) return;
#pragma unroll
        for (int t = 0; t < kSub; ++t) {
            const int p = pbase + res_tile * kCB + 32 * t + n;
            if (p < P) {
                const bool ok = (res_ok >> t) & 1u;
                scores[(size_t)r * P + p] = ok ? res[t] : -INFINITY;
                cand[(size_t)r * P + p] = ok ? 1 : 0;
            }
        }
    };

    for (int it = 0; it < ntiles; ++it) {
        const uint32_t fl = fl_next;
        store_results();
        if (it + 1 < ntiles) {
            issue_tile(it + 1);
            fl_next = load_flags(it + 1);
        }
        const uint8_t *T = ktile[it & 1];
#pragma unroll
        for (int t = 0; t < kSub; ++t) {
            const int pl = 32 * t + n;  // pool of this lane within the tile
            const uint8_t *Tt = T + 32 * t * kRowBytes;  // (pl & mask) == (n & mask): koff holds
            f32x16 acc0 = {}, acc1 = {};
#pragma unroll
            for (int st = 0; st < kSteps; ++st) {
                u32x4 kb;
                if constexpr (FP8) {  // 16 fp8 channels feed two steps
                    const u32x4 raw = *reinterpret_cast<const u32x4 *>(Tt + koff[st >> 1]);
                    kb = (st & 1) ? e4m3x8_to_bf16x8(raw.z, raw.w) : e4m3x8_to_bf16x8(raw.x, raw.y);
                } else {
                    kb = *reinterpret_cast<const u32x4 *>(Tt + koff[st]);
                }
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[0][st]), as_bf16x8(kb), acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[1][st]), as_bf16x8(kb), acc1, 0, 0, 0);
            }
            const float f = FP8 ? scale * ks_s[it & 1][pl] : scale;
            const float tot0 = f * add_xor32(relu_weighted(acc0, wr0, f));
            const float tot1 = f * add_xor32(relu_weighted(acc1, wr1, f));
            const float tot = half ? tot1 : tot0;
            res[t] = tot == 0.0f ? 0.0f : tot;
        }
        const int pt = pbase + it * kCB + n;
        const int lim = half ? lim1 : lim0;
        res_ok = 0u;
#pragma unroll
        for (int t = 0; t < kSub; ++t) res_ok |= (((fl >> t) & 1u) && pt + 32 * t < lim) ? 1u << t : 0u;
        res_tile = it;
        wait_vm<0>();     // tile it+1 has landed (and the stores issued above are done)
        __syncthreads();  // ... for every wave; buffer it&1 is free for tile it+2
    }
    store_results();
}

template <int D, bool FP8>
hipError_t launch_rowblock_d(int Q, int P, int Hi, int KP, int first_key, float scale,
                             const uint16_t *q, const float *w, const int32_t *row_seq,
                             const int32_t *row_pos, const void *keys, const float *key_scales,
                             const uint8_t *pool_valid, float *scores, uint8_t *cand,
                             hipStream_t stream) {
    hipLaunchKernelGGL((index_scores_rowblock_kernel<D, FP8>),
                       dim3((Q + kRB - 1) / kRB, (P + kCB * kTiles - 1) / (kCB * kTiles)), dim3(kRBThreads), 0, stream,
                       Q, P, Hi, KP, first_key, scale, q, w, row_seq, row_pos, keys, key_scales,
                       pool_valid, scores, cand);
    return hipGetLastError();
}

template <int D, bool FP8, int TPW>
hipError_t launch_valid_d(int Q, int B, int P, int Hi, int KP, int first_key, float scale,
                          const uint16_t *q, const float *w, const int32_t *row_seq,
                          const int32_t *row_pos, const void *keys, const float *key_scales,
                          const uint8_t *pool_valid, float *scores, uint8_t *cand,
                          hipStream_t stream) {
    constexpr int chunk = (kThreads / kWave) * TPW * 32;
    const int chunks = (P + chunk - 1) / chunk;
    const long long total = (long long)Q * chunks;
    if (total > INT32_MAX) return hipErrorInvalidValue;
    // Blocks resident at once on this device, for each form (cached per device).
    static std::mutex mu;
    static int resident[64][2] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (resident[dev][0] == 0) {
            int one = 0, walk = 0, cus = 0;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &one, reinterpret_cast<const void *>(&index_scores_valid_kernel<D, FP8, TPW, false>), kThreads, 0);
            if (e == hipSuccess)
                e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &walk, reinterpret_cast<const void *>(&index_scores_valid_kernel<D, FP8, TPW, true>), kThreads, 0);
            if (e == hipSuccess) e = device_cu_count(&cus);
            if (e != hipSuccess) return e;
            resident[dev][0] = std::max(1, one) * std::max(1, cus);
            resident[dev][1] = std::max(1, walk) * std::max(1, cus);
        }
    }
    if (total <= resident[dev][0])
        hipLaunchKernelGGL((index_scores_valid_kernel<D, FP8, TPW, false>), dim3((int)total), dim3(kThreads), 0,
                           stream, Q, chunks, B, P, Hi, KP, first_key, scale, q, w, row_seq, row_pos,
                           keys, key_scales, pool_valid, scores, cand);
    else
        hipLaunchKernelGGL((index_scores_valid_kernel<D, FP8, TPW, true>), dim3(resident[dev][1]),
                           dim3(kThreads), 0, stream, Q, chunks, B, P, Hi, KP, first_key, scale, q, w,
                           row_seq, row_pos, keys, key_scales, pool_valid, scores, cand);
    return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_d(int Q, int B, int P, int Hi, int KP, int first_key, float scale,
                    const uint16_t *q, const float *w, const int32_t *row_seq,
                    const int32_t *row_pos, const void *keys, const float *key_scales,
                    const int32_t *ids, const int32_t *n_valid, float *scores, uint8_t *cand,
                    hipStream_t stream) {
    const int chunks = P > 0 ? (P + kChunk - 1) / kChunk : 1;
    hipLaunchKernelGGL((index_scores_kernel<D, FP8>), dim3(Q, chunks), dim3(kThreads), 0, stream,
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

hipError_t launch_index_scores_valid(int Q, int B, int P, int Hi, int D, int KP, int first_key,
                                     float scale, const uint16_t *q, const float *w,
                                     const int32_t *row_seq, const int32_t *row_pos,
                                     const void *keys, bool key_fp8, const float *key_scales,
                                     const uint8_t *pool_valid, float *scores, uint8_t *cand,
                                     hipStream_t stream) {
    if (Q == 0 || P == 0) return hipSuccess;
    // Many rows of one sequence (prefill): the row-blocked product, keys read once per 16 rows.
    if (B == 1 && Q >= kRB) {
#define DSA_ISR_CASE(d)                                                                         \
        if (D == d)                                                                             \
            return key_fp8 ? launch_rowblock_d<d, true>(Q, P, Hi, KP, first_key, scale, q, w,   \
                                                        row_seq, row_pos, keys, key_scales,     \
                                                        pool_valid, scores, cand, stream)       \
                           : launch_rowblock_d<d, false>(Q, P, Hi, KP, first_key, scale, q, w,  \
                                                         row_seq, row_pos, keys, key_scales,    \
                                                         pool_valid, scores, cand, stream);
        DSA_ISR_CASE(32)
        DSA_ISR_CASE(64)
        DSA_ISR_CASE(128)
#undef DSA_ISR_CASE
    }
    // Two tiles a wave for fp8 keys (256 pool slots a block) and one for bf16 (128): rows of
    // very different lengths leave only some ranges with candidates, and smaller ranges spread
    // that work over more compute units (measured: fp8 at 128K contexts 8.6 us against 9.5 us
    // with four tiles; bf16 14.5 us against 15.0 us with two).
#define DSA_ISV_CASE(d)                                                                          \
    if (D == d)                                                                                  \
        return key_fp8 ? launch_valid_d<d, true, 2>(Q, B, P, Hi, KP, first_key, scale, q, w,     \
                                                    row_seq, row_pos, keys, key_scales,          \
                                                    pool_valid, scores, cand, stream)            \
                       : launch_valid_d<d, false, 1>(Q, B, P, Hi, KP, first_key, scale, q, w,    \
                                                     row_seq, row_pos, keys, key_scales,         \
                                                     pool_valid, scores, cand, stream);
    DSA_ISV_CASE(32)
    DSA_ISV_CASE(64)
    DSA_ISV_CASE(128)
#undef DSA_ISV_CASE
    return hipErrorInvalidValue;
}

}  // namespace dsa

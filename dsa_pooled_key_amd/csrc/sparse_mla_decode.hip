// sparse_mla_decode.hip -- absorbed-query NoPE MLA attention over the selected tokens.
//
// build.rs, "The transforms" 1 and 3: the query is absorbed into the 512-wide latent and the
// output stays in latent space ([heads, kv_lora_rank]); mod.rs: NoPE, a 512-wide latent,
// attention restricted to the expanded token ids, and the serve path reads those tokens
// through a block table with no sequence-length-sized buffer.
//
// Keys and values are the same latent rows, so each 32-token tile is gathered once from HBM
// straight into LDS (global_load_lds, no registers) in its storage format -- fp8 e4m3 rows of
// 512 bytes or bf16 rows of 1 KiB -- and read there by both products:
//   S^T = K . Q^T  on v_mfma_f32_16x16x32_bf16: wave w scores 16 tokens x 16 heads over all 512
//                  channels; its query fragment (64 registers) stays resident. fp8 rows are
//                  read 16 channels at a time and converted to bf16 in registers (exact).
//   O  += P . V    on v_mfma_f32_32x32x16_bf16: wave w owns 32 heads x 128 channels of the output
//                  accumulator (64 registers), reads P (bf16) from LDS and V down the token axis
//                  of the same tile with gfx950's LDS transpose reads (8-bit for fp8 rows, then
//                  converted; 16-bit for bf16 rows).
// The softmax is online with a lazily moved reference maximum per head. For fp8 the per-token
// scale multiplies the logit and the probability, so no rounding beyond bf16 P is added.
//
// Split over tokens: block (r, s, g) takes token slots [s*L, s*L + L) of row r for head group g.
// With one split the block writes out and lse directly; with several it writes (max, sum,
// unnormalised O) to the workspace and mla_combine merges them.
//
// Bytes per selected token: 1024 (bf16) or 516 (fp8 + scale) of latent, 4 of token id.
#include <mutex>

#include "dsa_device.hpp"
#include "dsa_launch.hpp"
#include "dsa_phase.hpp"

DSA_PHASE_TABLE(mla)

namespace dsa {

// Fixed device scratch for dsa_sparse_mla_decode_noalloc: the split partials live here instead
// of in a caller's workspace. Each GPU the library runs on holds its own copy for the life of
// the process. In host code this name is only a stand-in for the symbol; kernels get the device
// address that mla_noalloc_scratch() looks up.
__device__ __attribute__((aligned(256))) uint8_t scratch[kMlaNoallocScratchBytes];

hipError_t mla_noalloc_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

constexpr int kC = 512;
constexpr int kTile = 32;
constexpr int kThreads = 256;          // 4 waves
constexpr int kMaxSplit = kMlaMaxSplit;   // token slots one block resolves up front
constexpr int kMaxSplits = kMlaMaxSplits; // splits per (row, group)
constexpr int kPStride = kTile + 8;    // bf16 per P row (80 bytes: conflict-free row reads)
// Split partial per (row, group, split): max[32] and sum[32] (f32), then the unnormalised O of
// 32 heads x 512 channels in bf16 -- the precision of the P operand it was accumulated from --
// stored in accumulator order: 16-byte vector ((v*4 + nt)*2 + i8)*64 + lane holds
// acc[nt][8*i8 .. 8*i8 + 7] of lane `lane` of wave v.
constexpr int kPartHeader = 256;
constexpr int kPartBytes = kPartHeader + 32 * kC * 2;
// Partials are stored with the sc0 and sc1 cache-policy bits (written through to the memory
// side rather than held dirty in the writing XCD's L2): the main kernel's end then has little to
// write back before the combine can start, and the combine, whose blocks run on any XCD, reads
// them from there (45.6 against 46.4 us for the fp8_mixed_b32 step; streaming stores alone
// gave 45.9).
constexpr int kWriteThrough = 1 | 16;  // sc0 | sc1

// Tile geometry per storage format. A tile is 32 rows; rows arrive by 16-byte-a-lane DMA and
// keep their storage format in LDS. Chunk c (16 bytes) of row r sits at position c ^ swz(r);
// the two swizzles were chosen by measuring each read pattern below on gfx950 (all four run
// at the conflict-free rate of their instruction).
template <bool FP8>
struct Geo {
    static constexpr int kRowBytes = FP8 ? 512 : 1024;
    static constexpr int kTileBytes = kTile * kRowBytes;
    static constexpr int kStages = FP8 ? 4 : 2;            // tiles resident in the ring
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows one wave-wide load covers
    static constexpr int kLoads = 8 / kRowsPerLoad;        // row loads per wave per tile (8 rows)
    static constexpr int kLoadsT = kLoads + (FP8 ? 1 : 0); // plus the rows' fp8 scales
    static constexpr int kLanesPerRow = kWave / kRowsPerLoad;
};
template <bool FP8>
__device__ __forceinline__ int swz(int r) {
    return FP8 ? ((r & 15) ^ ((r >> 4) & 1)) : (((r & 7) << 1) | ((r >> 3) & 1));
}
// The softmax keeps a reference maximum per head and moves it only when a tile's maximum
// exceeds it by more than this many (natural-log) units, so the accumulator is rescaled on
// few tiles; unnormalised weights stay below e^8.
constexpr float kRescaleSlack = 8.0f;

// Block barrier that orders LDS traffic only (outstanding tile loads keep flowing).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <class T>
__device__ __forceinline__ T lds_load(const uint8_t *base, uint32_t off) {
    return *reinterpret_cast<const T *>(base + off);
}

// Team = 4 waves working one token split. Wave v scores tile rows 16*(v>>1).. x heads
// 16*(v&1).. and accumulates O for channels 128v..128v+127 of all 32 heads of group g.
// A block holds TEAMS teams on consecutive splits of the same row and head group: they share
// the staged query rows and every barrier, and merge their (max, sum, O) in LDS at the end,
// so the block leaves one partial (or, covering the whole row, the output itself).
//
// Query channels are permuted inside each MFMA step (the contraction order is free as long
// as both operands agree): step s, lane group k (= lane>>4) covers channels
// 64*(s>>1) + 16k + 8*(s&1) .. +7, so one 16-byte read of an fp8 row feeds two steps.
template <bool FP8, bool PAGED, int TEAMS>
__global__ __launch_bounds__(kThreads * TEAMS) __attribute__((amdgpu_waves_per_eu(2))) void sparse_mla_kernel(
    int W, int H, int B, int splits, int split_len, float sm_scale,
    const uint16_t *__restrict__ q_abs, const int32_t *__restrict__ token_ids,
    const int32_t *__restrict__ row_seq, const void *__restrict__ kv,
    const float *__restrict__ kv_scales, long long kv_rows, int S,
    const int32_t *__restrict__ block_table, int max_blocks, int block_size,
    float *__restrict__ out, float *__restrict__ lse, float *__restrict__ ws) {
    using G_ = Geo<FP8>;
    constexpr int NS = G_::kStages;
    constexpr int RB = G_::kRowBytes;

    static_assert(TEAMS == 1 || TEAMS == 2, "one or two teams per block");
    // One set per team.
    __shared__ __attribute__((aligned(16))) uint8_t ring_all[TEAMS][NS * G_::kTileBytes];
    __shared__ __attribute__((aligned(16))) uint16_t pl_all[TEAMS][32 * kPStride];
    __shared__ __attribute__((aligned(16))) int rows_all[TEAMS][kMaxSplit];
    // fp8 scales of each resident tile: wave w's 8 rows at [stage][w][0..7] (64 per wave land).
    __shared__ __attribute__((aligned(16))) float sc_all[TEAMS][FP8 ? NS : 1][4][kWave];
    __shared__ float red_all[TEAMS][4][16];
    __shared__ float alpha_all[TEAMS][32];
    __shared__ float msum_all[TEAMS][32];
    __shared__ float lsum_all[TEAMS][32];
    __shared__ int last_all[TEAMS][4];
    __shared__ int rescale_all[TEAMS][2];
    __shared__ __attribute__((aligned(16))) float mf_s[TEAMS][32];  // per-head merge factors

    DSA_PHASE(2, 0);  // block start
    const int r = blockIdx.x;
    const int tm = threadIdx.x / kThreads;  // team
    const int split = blockIdx.y * TEAMS + tm;
    const int g = blockIdx.z;
    const int G = gridDim.z;
    const int tid = threadIdx.x % kThreads;  // thread within the team
    const int lane = tid & (kWave - 1);
    const int v = tid / kWave;  // wave 0..3 of the team
    uint8_t *const ring = ring_all[tm];
    uint16_t *const pl = pl_all[tm];
    int *const rows_s = rows_all[tm];
    float(*const sc_ring)[4][kWave] = sc_all[tm];
    float(*const red)[16] = red_all[tm];
    float *const alpha_s = alpha_all[tm];
    float *const msum_s = msum_all[tm];
    float *const lsum_s = lsum_all[tm];
    int *const last_w = last_all[tm];
    int *const rescale_s = rescale_all[tm];
    const int lg = lane >> 4;   // 16-lane group
    const int b = row_seq[r];
    const bool row_ok = b >= 0 && b < B;
    const int s0 = split * split_len;
    const int n_slots = max(0, min(split_len, W - s0));
    const uint8_t *kvb = static_cast<const uint8_t *>(kv);

    // The block's 32 query rows (1 KiB each) are staged once through LDS, in the upper half of
    // team 0's ring, which no tile uses before every wave of the block has taken its fragment:
    // wave w of the block fetches 8/TEAMS heads from (8/TEAMS)w on, chunk c of head row h at
    // position c ^ swz<false>(h). fp8 issues the copies with tile 0's, after the token ids and
    // table entries have landed, so those small loads do not queue behind them (47.3 against
    // 47.7 us for the fp8_mixed_b32 step); bf16 issues them first (later, its X128 decode and
    // prefill attention took 3% longer).
    uint8_t *const qlds = ring_all[0] + 32768;
    const int qk_head_local = 16 * (v & 1) + (lane & 15);
    const int qk_head = g * 32 + qk_head_local;
    constexpr int kQHeads = 8 / TEAMS;
    auto stage_q = [&]() {
#pragma unroll
        for (int k = 0; k < kQHeads; ++k) {
            const int hl = kQHeads * (int)(threadIdx.x / kWave) + k;
            if (g * 32 + hl < H)
                dma16(reinterpret_cast<const uint8_t *>(q_abs + ((size_t)r * H + g * 32 + hl) * kC) +
                          16 * (lane ^ swz<false>(hl)),
                      __builtin_amdgcn_readfirstlane(lds_offset(qlds + hl * 1024)));
        }
    };
    if constexpr (!FP8) stage_q();
    // ---- DMA: wave v fetches rows 8v..8v+7 of every tile (and, for fp8, their scales). A slot
    // without a token fetches latent row 0 (finite data; its weight is zero).
    const int dma_rl = lane / G_::kLanesPerRow;                    // row within one load
    const uint32_t dma_col = 16 * ((lane % G_::kLanesPerRow));     // byte position in the row
    // The wave's 8 latent rows of tile t (and, for fp8, lane&7's row for the scale copy) are
    // read from rows_s first; issue_rows() then starts the copies.
    struct TileRows {
        int4 a, b;
        int srow;
    };
    auto read_rows = [&](int t) {
        TileRows tr;
        tr.a = *reinterpret_cast<const int4 *>(rows_s + t * kTile + 8 * v);
        tr.b = *reinterpret_cast<const int4 *>(rows_s + t * kTile + 8 * v + 4);
        tr.srow = FP8 ? rows_s[t * kTile + 8 * v + (lane & 7)] : 0;
        return tr;
    };
    auto issue_rows = [&](int t, const TileRows &tr) {
        uint8_t *stage = ring + (t % NS) * G_::kTileBytes + 8 * v * RB;
        const int rws[8] = {tr.a.x, tr.a.y, tr.a.z, tr.a.w, tr.b.x, tr.b.y, tr.b.z, tr.b.w};
#pragma unroll
        for (int k = 0; k < G_::kLoads; ++k) {
            const int rl = k * G_::kRowsPerLoad;  // first row of this load within the wave's 8
            int prow = G_::kRowsPerLoad == 2 ? (dma_rl ? rws[rl + 1] : rws[rl]) : rws[rl];
            prow = max(prow, 0);
            const int rr = 8 * v + rl + dma_rl;  // row within the tile
            const uint8_t *src = kvb + (size_t)prow * RB + (dma_col ^ (uint32_t)(16 * swz<FP8>(rr)));
            dma16(src, __builtin_amdgcn_readfirstlane(lds_offset(stage + k * 1024)));
        }
        if constexpr (FP8)
            dma4(kv_scales + max(tr.srow, 0),
                 __builtin_amdgcn_readfirstlane(lds_offset(&sc_ring[t % NS][v][0])));
    };
    auto issue = [&](int t) { issue_rows(t, read_rows(t)); };

    // ---- prologue: wave v resolves the slots its own DMA fetches -- slot t*32 + 8v + j of
    // every tile t -- to latent rows (or -1) and issues the first tiles at once; it reads
    // back only the entries it wrote, so no barrier precedes the loads. Slots past n_slots up
    // to the tile boundary read as "no token", so the tile loop needs no bounds test.
    const int n_ptiles = (n_slots + kTile - 1) / kTile;
    int my_last = -1;
    for (int t0 = 0; t0 < n_ptiles; t0 += 8) {
        const int t = t0 + (lane >> 3);
        if (t < n_ptiles) {
            const int i = t * kTile + 8 * v + (lane & 7);
            const int tok = i < n_slots ? token_ids[(size_t)r * W + s0 + i] : -1;
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
            rows_s[i] = (int)row;
            if (row >= 0) my_last = i;
        }
    }
    // Tiles issued ahead: fp8 keeps two tiles in flight beyond the one being scored (a fourth
    // stage holds the tile whose products are still pending); bf16 keeps one tile in flight
    // and refills after the barrier that opens tile t. A tile without tokens fetches row 0,
    // so nothing is fetched from an empty latent buffer. The prologue issues only tile 0: in
    // the chip-wide burst of first tiles each team's tile 0 then lands before any tile 1
    // (fp8 issues tile 1 after the prologue barrier, 29.9 against 30.3 us for the stage on
    // fp8_mixed_b32).
    DSA_PHASE(2, 1);  // token ids and latent rows resolved
    if constexpr (FP8) stage_q();  // the query rows with tile 0
    const int pre = kv_rows > 0 ? min(n_ptiles, 1) : 0;
    for (int t = 0; t < pre; ++t) issue(t);
    my_last = (int)wave_reduce_u32((uint32_t)my_last,
                                   [](uint32_t a, uint32_t c) { return (int)a > (int)c ? a : c; });
    if (lane == 0) last_w[v] = my_last;
    if (tid < 2) rescale_s[tid] = 0;
    // The query rows, ids and table entries have landed (loads complete in order); fp8 also
    // waits for its own rows of tile 0. The barrier publishes both.
    if (FP8 || pre == 0) wait_vm<0>();
    else wait_vm<G_::kLoadsT>();
    __syncthreads();
    DSA_PHASE(2, 2);  // query rows and tile 0 landed, prologue barrier passed
    const int last = max(max(last_w[0], last_w[1]), max(last_w[2], last_w[3]));
    const int n_tiles = (last + kTile) / kTile;  // through the last slot with a token
    // The teams step through n_iter tiles together, since the barriers are the block's; a team
    // past its own last tile keeps only the barriers.
    int n_iter = n_tiles;
    if constexpr (TEAMS == 2) {
        const int *lo = last_all[tm ^ 1];
        n_iter = max(n_iter, (max(max(lo[0], lo[1]), max(lo[2], lo[3])) + kTile) / kTile);
    }

    if constexpr (FP8) {
        if (kv_rows > 0 && 1 < n_tiles) issue(1);
    }

    // Query fragment for S^T = K Q^T (B operand): head column lane&15 of this wave's 16; step st,
    // lane group lg holds channels 64(st>>1) + 16lg + 8(st&1) .. +7 (chunk 8(st>>1) + 2lg + (st&1)).
    u32x4 qf[16];
    {
        const int sw = swz<false>(qk_head_local);
#pragma unroll
        for (int st = 0; st < 16; ++st) {
            const int c = 8 * (st >> 1) + 2 * lg + (st & 1);
            qf[st] = qk_head < H ? lds_load<u32x4>(qlds, (uint32_t)(qk_head_local * 1024 + 16 * (c ^ sw)))
                                 : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // ---- LDS read offsets, hoisted out of the tile loop (per lane, within one tile).
    // QK operand: row tb + (lane&15). fp8: read jj (0..7) takes chunk 4jj + lg (two steps);
    // bf16: step st takes chunk 8(st>>1) + 2lg + (st&1). Both: base + 64/256 * (...) forms.
    const int tb = 16 * (v >> 1);
    const int qk_row = tb + (lane & 15);
    const int qk_sw = swz<FP8>(qk_row);
    uint32_t qk_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (FP8)  // chunk 4jj + lg, jj = 4a + j: position 16a + 4(j ^ sw>>2) + (lg ^ sw&3)
            qk_off[j] = (uint32_t)(qk_row * RB + 16 * (4 * (j ^ (qk_sw >> 2)) + (lg ^ (qk_sw & 3))));
        else  // chunk 8(st>>1) + 2lg + (st&1), st = 4a + j: position 16a + ((8(j>>1) + 2lg + (j&1)) ^ sw)
            qk_off[j] = (uint32_t)(qk_row * RB + 16 * ((8 * (j >> 1) + 2 * lg + (j & 1)) ^ qk_sw));
    }
    // V operand. fp8 (one 8-bit transpose read per fragment): source lane s of group lg reads
    // row 16ks + 8(lg>>1) + (s>>1), channels 128v + 32nt + 16(lg&1) + 8(s&1) .. +7.
    // bf16 (two 16-bit transpose reads): row 16ks + 8(lg>>1) + (s>>2) + 4h, channels
    // 128v + 32nt + 16(lg&1) + 4(s&3) .. +3.
    const int vs = lane & 15;
    uint32_t v_off[2][4];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            if constexpr (FP8) {  // x = ks
                const int row = 16 * x + 8 * (lg >> 1) + (vs >> 1);
                const int c = 8 * v + 2 * nt + (lg & 1);
                v_off[x][nt] = (uint32_t)(row * RB + 16 * (c ^ swz<true>(row)) + 8 * (vs & 1));
            } else {  // x = h; ks adds 16 rows (same swizzle)
                const int row = 8 * (lg >> 1) + (vs >> 2) + 4 * x;
                const int ch = 128 * v + 32 * nt + 16 * (lg & 1) + 4 * (vs & 3);
                v_off[x][nt] = (uint32_t)(row * RB + 16 * ((ch >> 3) ^ swz<false>(row)) + 2 * (ch & 7));
            }
        }

    float m_ref = -INFINITY;  // reference maximum of head qk_head
    float l_run = 0.0f;       // this lane's share of the running sum
    f32x16 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x16{};

    // ---- phases of one tile
    // Scores S^T[token][head] for this wave's 16 tokens x 16 heads (two MFMA chains), scaled
    // and masked into x; sc gets the rows' fp8 scales (1 for bf16, 0 where there is no token).
    // The wave's maxima per head go to red[v].
    // Slots tb + 4lg .. +3 of tile t (16-byte aligned) and, for fp8, their rows' scales (rows
    // tb + 4lg .. +3 were fetched by wave (tb + 4lg) >> 3).
    auto score_rows = [&](int t) {
        return *reinterpret_cast<const int4 *>(rows_s + t * kTile + tb + lg * 4);
    };
    auto score_scales = [&](int t) {
        f32x4 sv = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (FP8) {
            const int rr = tb + lg * 4;
            sv = *reinterpret_cast<const f32x4 *>(&sc_ring[t % NS][rr >> 3][rr & 7]);
        }
        return sv;
    };
    auto score_epilogue = [&](const f32x4 &sa, const f32x4 &sb, const int4 &rw, const f32x4 &sv,
                              float (&x)[4], float (&sc)[4]) {
        const int rwa[4] = {rw.x, rw.y, rw.z, rw.w};
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = rwa[i] >= 0;
            sc[i] = ok ? sv[i] : 0.0f;
            x[i] = ok ? (sa[i] + sb[i]) * (sm_scale * sc[i]) : -INFINITY;
            tmax = fmaxf(tmax, x[i]);
        }
        tmax = max_xor32(max_xor16(tmax));
        if (lane < 16) red[v][lane] = tmax;
    };
    auto scores = [&](int t, float (&x)[4], float (&sc)[4]) {
        const uint8_t *T = ring + (t % NS) * G_::kTileBytes;
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const u32x4 raw = lds_load<u32x4>(T, qk_off[jj & 3] + 256 * (jj >> 2));
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(e4m3x8_to_bf16x8(raw.x, raw.y)),
                                                              as_bf16x8(qf[2 * jj]), sa, 0, 0, 0);
                sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(e4m3x8_to_bf16x8(raw.z, raw.w)),
                                                              as_bf16x8(qf[2 * jj + 1]), sb, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int st = 0; st < 16; st += 2) {
                const u32x4 a0 = lds_load<u32x4>(T, qk_off[st & 3] + 256 * (st >> 2));
                const u32x4 a1 = lds_load<u32x4>(T, qk_off[(st + 1) & 3] + 256 * ((st + 1) >> 2));
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qf[st]), sa, 0, 0, 0);
                sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qf[st + 1]), sb, 0, 0, 0);
            }
        }
        const int4 rw = score_rows(t);
        const f32x4 sv = score_scales(t);
        score_epilogue(sa, sb, rw, sv, x, sc);
    };
    // After the maxima are exchanged: move the reference maximum if needed, write P (bf16,
    // fp8 scale folded in) and the rescale factors of tile t (flag parity t&1).
    auto softmax = [&](int t, const float (&x)[4], const float (&sc)[4]) {
        const int par = t & 1;
        const float m_tile = fmaxf(red[v][lane & 15], red[v ^ 2][lane & 15]);
        float alpha = 1.0f;
        if (m_tile > m_ref + kRescaleSlack) {  // also true for the first tile with a token
            alpha = m_ref == -INFINITY ? 0.0f : fast_exp(m_ref - m_tile);
            m_ref = m_tile;
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = x[i] == -INFINITY ? 0.0f : fast_exp(x[i] - m_ref);
        l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        *reinterpret_cast<u32x2 *>(pl + qk_head_local * kPStride + tb + lg * 4) =
            u32x2{pack_bf16x2(p[0] * sc[0], p[1] * sc[1]), pack_bf16x2(p[2] * sc[2], p[3] * sc[3])};
        if (v < 2 && lane < 16) {
            alpha_s[qk_head_local] = alpha;
            if (alpha != 1.0f) rescale_s[par] = 1;
        }
        // The other parity's flag was last read by the products of tile t-1, which every wave
        // finished before the barrier this phase follows; it is set again for tile t+1.
        if (v == 0 && lane == 0) rescale_s[par ^ 1] = 0;
    };
    // O[head][channel] += P . V over tile t's 32 tokens; this wave: 128 channels. V fragments
    // come down the token axis through the LDS transpose reads.
    auto rescale_acc = [&]() {
        float al[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) al[i] = alpha_s[8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nt][i] *= al[i];
    };
    auto products = [&](int t) {
        const uint8_t *T = ring + (t % NS) * G_::kTileBytes;
        if (rescale_s[t & 1]) rescale_acc();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(pl + (lane & 31) * kPStride + 16 * ks +
                                                             (lane >> 5) * 8);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                u32x4 vv;
                if constexpr (FP8) {
                    const u32x2 raw = lds_read_tr8(T + v_off[ks][nt]);
                    vv = e4m3x8_to_bf16x8(raw.x, raw.y);
                } else {
                    const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t *>(
                        T + v_off[0][nt] + 16 * RB * ks));
                    const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t *>(
                        T + v_off[1][nt] + 16 * RB * ks));
                    vv = u32x4{lo.x, lo.y, hi.x, hi.y};
                }
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(vv),
                                                                  acc[nt], 0, 0, 0);
            }
        }
    };

    if constexpr (FP8) {
        // Software-pipelined: the scores of tile t and the products of tile t-1 interleave.
        // Iteration t first refills the stage of tile t-2 (its products ended before barrier C
        // of tile t-1) with tile t+2. Per tile two barriers: B (maxima exchanged) and C (P of
        // tile t visible, tile t+1 resident). Before B a wave takes its P operand of tile t-1
        // into registers and applies tile t-1's rescale, then scores tile t; after B the
        // products of tile t-1 run beside the softmax of tile t, whose P, alpha and flag
        // writes therefore touch nothing those products still read.
        auto pv = [&](int t, const u32x4 (&pa)[2]) {  // O += P(t) V(t), P already in registers
            const uint8_t *TP = ring + (t % NS) * G_::kTileBytes;
            u32x2 vr[2][4];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) vr[ks][nt] = lds_read_tr8(TP + v_off[ks][nt]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(pa[ks]), as_bf16x8(e4m3x8_to_bf16x8(vr[ks][nt].x, vr[ks][nt].y)),
                        acc[nt], 0, 0, 0);
        };
        if (n_iter > 0) {
            float x[4], sc[4];
            if (n_tiles > 0) scores(0, x, sc);
            lds_barrier();  // B; every wave holds its query fragment, so stage 2 is free
            if (n_tiles > 0) {
                if (2 < n_tiles) issue(2);
                softmax(0, x, sc);
                if (2 < n_tiles) wait_vm<G_::kLoadsT>();
                else wait_vm<0>();
            }
            lds_barrier();  // C
        }
        DSA_PHASE(2, 3);  // first tile done
        // Iteration t, before B: every LDS operand of the refill, of tile t-1's P and of the
        // scores of tile t is requested before the first is used, so their latencies overlap
        // one another and the MFMA work instead of adding up.
        auto step = [&](int t, float (&x)[4], float (&sc)[4], u32x4 (&pa)[2]) {
            const bool refill = t + 2 < n_tiles;
            const uint8_t *TS = ring + (t % NS) * G_::kTileBytes;
            TileRows nr{};
            if (refill) nr = read_rows(t + 2);
            const int resc = rescale_s[(t - 1) & 1];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                pa[ks] = *reinterpret_cast<const u32x4 *>(pl + (lane & 31) * kPStride + 16 * ks +
                                                          (lane >> 5) * 8);
            u32x4 kr[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) kr[jj] = lds_load<u32x4>(TS, qk_off[jj & 3] + 256 * (jj >> 2));
            const int4 rw = score_rows(t);
            const f32x4 sv = score_scales(t);
            __builtin_amdgcn_sched_barrier(0);
            if (refill) issue_rows(t + 2, nr);
            if (resc) rescale_acc();
            f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(e4m3x8_to_bf16x8(kr[jj].x, kr[jj].y)),
                                                              as_bf16x8(qf[2 * jj]), sa, 0, 0, 0);
                sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(e4m3x8_to_bf16x8(kr[jj].z, kr[jj].w)),
                                                              as_bf16x8(qf[2 * jj + 1]), sb, 0, 0, 0);
            }
            score_epilogue(sa, sb, rw, sv, x, sc);
        };
        for (int t = 1; t < n_iter; ++t) {
            float x[4], sc[4];
            if (t < n_tiles) {
                u32x4 pa[2];
                step(t, x, sc, pa);
                lds_barrier();  // B
                softmax(t, x, sc);
                pv(t - 1, pa);
                if (t + 2 < n_tiles) wait_vm<G_::kLoadsT>();  // tile t+1 landed, t+2 may fly
                else wait_vm<0>();
                lds_barrier();  // C
            } else {
                if (t == n_tiles) products(t - 1);  // the team's last tile
                lds_barrier();  // B
                lds_barrier();  // C
            }
        }
        if (n_tiles > 0 && n_tiles == n_iter) products(n_tiles - 1);
        DSA_PHASE(2, 4);  // every tile done
    } else {
        // bf16: one tile in flight (two 32 KiB stages); barrier A opens each tile once it is
        // resident and the stage of tile t-1 is free for tile t+1 (for t = 0: the query rows
        // in stage 1 have been read by every wave).
        for (int t = 0; t < n_iter; ++t) {
            float x[4], sc[4];
            const bool act = t < n_tiles;
            wait_vm<0>();
            lds_barrier();  // A
            if (act) {
                if (t + 1 < n_tiles) issue(t + 1);
                scores(t, x, sc);
            }
            lds_barrier();  // B
            if (act) softmax(t, x, sc);
            lds_barrier();  // C
            if (act) products(t);
        }
        DSA_PHASE(2, 4);  // every tile done
    }

    wait_vm<0>();  // a tile fetched ahead but past the last token still lands in LDS first
    // ---- finish: per-head sums (two waves score each head), then out or the split partial
    l_run = add_xor32(add_xor16(l_run));
    __syncthreads();
    if (lane < 16) red[v][lane] = l_run;
    __syncthreads();
    if (v < 2 && lane < 16) {
        lsum_s[qk_head_local] = red[v][lane] + red[v + 2][lane];
        msum_s[qk_head_local] = m_ref;
    }
    __syncthreads();

    if constexpr (TEAMS == 2) {
        // Team 1 hands its accumulator to team 0 through its own ring (idle now: its tiles have
        // landed and been used), f32 in accumulator order. Per head the merged maximum M, the
        // factors e^(m - M) (0 for a team without tokens) and the merged sum are formed once.
        f32x4 *xch = reinterpret_cast<f32x4 *>(ring_all[1]);
        if (tm == 1) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4)
                    xch[((v * 4 + nt) * 4 + i4) * kWave + lane] =
                        f32x4{acc[nt][4 * i4], acc[nt][4 * i4 + 1], acc[nt][4 * i4 + 2], acc[nt][4 * i4 + 3]};
        }
        if (threadIdx.x < 32) {
            const int h = threadIdx.x;
            const float ma = msum_all[0][h], mb = msum_all[1][h];
            const float la = lsum_all[0][h], lb = lsum_all[1][h];
            float M = -INFINITY;
            if (la > 0.0f) M = ma;
            if (lb > 0.0f) M = fmaxf(M, mb);
            const float fa = la > 0.0f ? fast_exp(ma - M) : 0.0f;
            const float fb = lb > 0.0f ? fast_exp(mb - M) : 0.0f;
            mf_s[0][h] = fa;
            mf_s[1][h] = fb;
            msum_all[0][h] = M;
            lsum_all[0][h] = la * fa + lb * fb;
        }
        __syncthreads();
        if (tm == 1) return;
        const int m0 = 4 * (lane >> 5);  // heads m0 + 8j .. +3 for element group j
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 fa = *reinterpret_cast<const f32x4 *>(&mf_s[0][8 * i4 + m0]);
            const f32x4 fb = *reinterpret_cast<const f32x4 *>(&mf_s[1][8 * i4 + m0]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const f32x4 o = xch[((v * 4 + nt) * 4 + i4) * kWave + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[nt][4 * i4 + e] = acc[nt][4 * i4 + e] * fa[e] + o[e] * fb[e];
            }
        }
    }

    DSA_PHASE(2, 5);  // teams merged
    // The block's result: out and lse when it covers the whole row, else partial blockIdx.y.
    const int parts = gridDim.y;
    if (parts == 1) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int ch = 128 * v + 32 * nt + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                const int hg = g * 32 + m;
                const float L = lsum_s[m];
                if (hg < H) out[((size_t)r * H + hg) * kC + ch] = L > 0.0f ? acc[nt][i] / L : 0.0f;
            }
        }
        if (lse != nullptr && tid < 32 && g * 32 + tid < H) {
            const float L = lsum_s[tid];
            lse[(size_t)r * H + g * 32 + tid] = L > 0.0f ? msum_s[tid] + logf(L) : -INFINITY;
        }
    } else {
        uint8_t *part = reinterpret_cast<uint8_t *>(ws) + (((size_t)r * G + g) * parts + blockIdx.y) * kPartBytes;
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(part, kPartBytes);
        if (tid < 32) {
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, msum_s[tid]), rs, 4 * tid, 0,
                                                  kWriteThrough);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lsum_s[tid]), rs, 128 + 4 * tid, 0,
                                                  kWriteThrough);
        }
        // a block without tokens writes its zero O too (sum 0), so the merge needs no test
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i8 = 0; i8 < 2; ++i8) {
                const f32x16 &a = acc[nt];
                const u32x4 vec{pack_bf16x2(a[8 * i8], a[8 * i8 + 1]), pack_bf16x2(a[8 * i8 + 2], a[8 * i8 + 3]),
                                pack_bf16x2(a[8 * i8 + 4], a[8 * i8 + 5]), pack_bf16x2(a[8 * i8 + 6], a[8 * i8 + 7])};
                __builtin_amdgcn_raw_buffer_store_b128(
                    vec, rs, kPartHeader + 16 * (((v * 4 + nt) * 2 + i8) * kWave + lane), 0, kWriteThrough);
            }
    }
    DSA_PHASE(2, 6);  // result stores issued
}

// Merge the split partials of one (row, head group): block z = 4v + nt covers channels
// 128v + 32nt .. +31 of all 32 heads. Per head the splits' (max m_s, sum l_s) give
// M = max m_s, L = sum l_s e^(m_s - M) and the weights e^(m_s - M) / L; out = sum_s weight_s O_s,
// lse = M + log L. Splits without tokens (l_s = 0) get weight 0; their O is zero.
// NP (2..kMaxSplits) is the split count, a template parameter so that every load count is
// known at compile time.
template <int NP>
__global__ __launch_bounds__(128) void mla_combine_kernel(const int H, const uint8_t *__restrict__ ws,
                                                          float *__restrict__ out,
                                                          float *__restrict__ lse) {
    __shared__ __attribute__((aligned(16))) float wgt[NP][32];
    __shared__ float red4[4][32];
    DSA_PHASE(3, 0);
    const int r = blockIdx.x;
    const int g = blockIdx.y;
    const int G = gridDim.y;
    const int z = blockIdx.z;  // 4v + nt
    const int tid = threadIdx.x;
    const uint8_t *base = ws + ((size_t)r * G + g) * NP * kPartBytes;
    const int i8 = tid >> 6, lane = tid & 63;
    const int slot = (z * 2 + i8) * kWave + lane;   // 16-byte vector within O
    auto o_vec = [&](int s) {
        return reinterpret_cast<const u32x4 *>(base + (size_t)s * kPartBytes + kPartHeader)[slot];
    };
    // Every split's header and O vectors are fetched in one round trip, the headers first: with
    // the split count fixed at compile time the weights below wait only for the headers
    // (loads complete in order) while the O vectors are still in flight.
    // Weights: thread (head h, quarter q) takes splits q, q+4, ...; the four quarters meet in LDS.
    const int h = tid & 31, q = tid >> 5;
    constexpr int kPer = (NP + 3) / 4;
    float ms[kPer], ls[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int sp = q + 4 * j;
        ms[j] = -INFINITY;
        ls[j] = 0.0f;
        if (sp < NP) {
            const float *hd = reinterpret_cast<const float *>(base + (size_t)sp * kPartBytes);
            ms[j] = hd[h];
            ls[j] = hd[32 + h];
        }
    }
    u32x4 pre[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) pre[k] = o_vec(k);
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use of a header
    {
        float M = -INFINITY;
#pragma unroll
        for (int j = 0; j < kPer; ++j) M = ls[j] > 0.0f ? fmaxf(M, ms[j]) : M;
        red4[q][h] = M;
        __syncthreads();
        M = fmaxf(fmaxf(red4[0][h], red4[1][h]), fmaxf(red4[2][h], red4[3][h]));
        float L = 0.0f;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            ms[j] = ls[j] > 0.0f ? fast_exp(ms[j] - M) : 0.0f;
            L += ls[j] * ms[j];
        }
        __syncthreads();
        red4[q][h] = L;
        __syncthreads();
        L = (red4[0][h] + red4[1][h]) + (red4[2][h] + red4[3][h]);
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (q + 4 * j < NP) wgt[q + 4 * j][h] = ms[j] * inv;
        if (lse != nullptr && z == 0 && q == 0 && g * 32 + h < H)
            lse[(size_t)r * H + g * 32 + h] = L > 0.0f ? M + logf(L) : -INFINITY;
    }
    __syncthreads();
    const int m_lo = 16 * i8 + 4 * (lane >> 5);    // heads m_lo..m_lo+3 and m_lo+8..m_lo+11
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto accumulate = [&](int s, const u32x4 &val) {
        const f32x4 wl = *reinterpret_cast<const f32x4 *>(&wgt[s][m_lo]);
        const f32x4 wh = *reinterpret_cast<const f32x4 *>(&wgt[s][m_lo + 8]);
        const float w[8] = {wl[0], wl[1], wl[2], wl[3], wh[0], wh[1], wh[2], wh[3]};
        const uint32_t u[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float x = (c & 1) ? bf16_hi(u[c >> 1]) : bf16_lo(u[c >> 1]);
            o[c] = fmaf(x, w[c], o[c]);
        }
    };
#pragma unroll
    for (int k = 0; k < NP; ++k) accumulate(k, pre[k]);
    const int ch = 32 * z + (lane & 31);  // 128v + 32nt + (lane & 31)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int h = g * 32 + m_lo + (c & 3) + 8 * (c >> 2);
        if (h < H) __builtin_nontemporal_store(o[c], &out[((size_t)r * H + h) * kC + ch]);  // read by a later kernel
    }
    DSA_PHASE(3, 1);
}

template <int NP>
hipError_t launch_combine(int parts, int Q, int groups, int H, const uint8_t *ws, float *out,
                          float *lse, hipStream_t stream) {
    if constexpr (NP > kMaxSplits) {
        return hipErrorInvalidValue;
    } else {
        if (parts != NP) return launch_combine<NP + 1>(parts, Q, groups, H, ws, out, lse, stream);
        hipLaunchKernelGGL(mla_combine_kernel<NP>, dim3(Q, groups, 16), dim3(128), 0, stream, H, ws,
                           out, lse);
        return hipGetLastError();
    }
}

template <bool FP8, bool PAGED>
hipError_t launch_v(const MlaPlan &plan, int Q, int W, int H, int B, float sm_scale,
                    const uint16_t *q_abs, const int32_t *token_ids, const int32_t *row_seq,
                    const void *kv, const float *kv_scales, int64_t kv_rows, int S,
                    const int32_t *block_table, int max_blocks, int block_size, float *out,
                    float *lse, void *ws, hipStream_t stream) {
    const dim3 grid(Q, plan.parts, plan.groups);
    if (plan.teams == 2)
        hipLaunchKernelGGL((sparse_mla_kernel<FP8, PAGED, 2>), grid, dim3(2 * kThreads), 0, stream, W, H, B,
                           plan.splits, plan.split_len, sm_scale, q_abs, token_ids, row_seq, kv, kv_scales,
                           (long long)kv_rows, S, block_table, max_blocks, block_size, out, lse,
                           static_cast<float *>(ws));
    else
        hipLaunchKernelGGL((sparse_mla_kernel<FP8, PAGED, 1>), grid, dim3(kThreads), 0, stream, W, H, B,
                           plan.splits, plan.split_len, sm_scale, q_abs, token_ids, row_seq, kv, kv_scales,
                           (long long)kv_rows, S, block_table, max_blocks, block_size, out, lse,
                           static_cast<float *>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.parts == 1) return e;
    return launch_combine<2>(plan.parts, Q, plan.groups, H, static_cast<const uint8_t *>(ws), out,
                             lse, stream);
}

}  // namespace

// Split the token slots so that about 512 teams (two 4-wave teams per compute unit) run,
// with at least 64 slots per split, at most kMaxSplit slots per split and at most kMaxSplits
// (16) splits per row, so that the combine reads every partial in one round trip (a 2,048-slot
// row in 32 splits of 64 took 1.5 us more, most of it in the combine); a row that already gives
// enough teams is not split. Where the teams fill
// one or two waves of resident blocks (512 to 1024 of them), pairs of splits share a block
// (one partial per pair). Larger grids keep one team per block: two blocks on a compute unit
// then drift apart in phase, so one's prologue overlaps the other's streaming, which paired
// teams in lockstep would lose.
MlaPlan plan_sparse_mla(int Q, int W, int H) {
    MlaPlan p;
    p.groups = (H + 31) / 32;
    const long long wr = ((long long)W + kTile - 1) / kTile * kTile;
    const long long work = (long long)W * Q * p.groups;
    long long per = (work + 511) / 512;
    per = ((per + kTile - 1) / kTile) * kTile;
    if (per < 64) per = 64;
    const long long floor_len = ((wr + kMaxSplits - 1) / kMaxSplits + kTile - 1) / kTile * kTile;
    if (per < floor_len) per = floor_len;
    if (per > kMaxSplit) per = kMaxSplit;
    if (per > wr) per = wr;
    if (per < kTile) per = kTile;
    p.splits = W > 0 ? (int)((W + per - 1) / per) : 1;
    if (p.splits > 1) {
        per = ((W + p.splits - 1) / p.splits + kTile - 1) / kTile * kTile;
        p.splits = (int)((W + per - 1) / per);
    }
    p.split_len = (int)per;
    const long long teams = (long long)Q * p.groups * p.splits;
    p.teams = p.splits > 1 && teams >= 512 && teams <= 1024 ? 2 : 1;
    p.parts = (p.splits + p.teams - 1) / p.teams;
    p.ws_bytes = p.parts > 1 ? (size_t)Q * p.groups * p.parts * kPartBytes : 0;
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

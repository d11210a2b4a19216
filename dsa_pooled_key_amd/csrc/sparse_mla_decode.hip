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
//                  output accumulator (64 registers) and reads P (bf16) from LDS and V down
//                  the token axis of the same tile with gfx950's LDS transpose read.
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
constexpr int kThreads = 512;          // 8 waves: two teams of 4 on alternate tiles
constexpr int kMaxSplit = 1024;        // token slots one block resolves up front
constexpr int kMaxSplits = 64;         // splits per (row, group)
constexpr int kPStride = kTile + 8;    // bf16 per P row
constexpr int kPartFloats = 64 + 32 * kC;  // per (row, group, split): max[32], sum[32], O[32][512]

// Tiles of 32 latent rows. The working tile is bf16, one 1 KiB row per token, its 16-byte
// chunks XOR-swizzled (chunk c of row r at position c ^ swz_work(r)) so that the QK operand
// reads (16 rows, one chunk column) and the transposing V reads (4 rows, 4 chunk columns per
// 32 lanes) each touch distinct LDS banks. Rows arrive by global_load_lds_dwordx4 (16 bytes
// a lane, no registers): a bf16 latent lands directly in a ring of working tiles; an fp8
// latent lands in a ring of raw 512-byte rows (chunk c of row r at c ^ 8*(r&1)) and the
// wave that fetched a row converts it into the working tile, once per element.
__device__ __forceinline__ int swz_work(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
constexpr int kWorkRow = 1024;
constexpr int kWorkTile = kTile * kWorkRow;
constexpr int kRawRow = 512;
constexpr int kRawWave = 8 * kRawRow;  // the 8 rows of one tile one wave fetches
// The softmax keeps a reference maximum per head and moves it only when a tile's maximum
// exceeds it by more than this many (natural-log) units, so the accumulator is rescaled on
// few tiles; unnormalised weights stay below e^8.
constexpr float kRescaleSlack = 8.0f;

// One 16-byte-a-lane global -> LDS copy (global_load_lds_dwordx4): lane l's 16 bytes land
// at lds_base + 16*l. Issued as inline assembly so the compiler does not treat it as an LDS
// write and order every later LDS read behind it; completion is tracked by the explicit
// vmcnt waits below (loads complete in order, so the compiler's own waits stay correct).
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)(p);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
// The builtin form lets the compiler's own wait insertion see these waits.
template <int N>
__device__ __forceinline__ void wait_vm() {  // at most N vector-memory loads outstanding
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

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

// Block = 8 waves in two teams. Team tm (waves 4tm..4tm+3) processes tiles tm, tm+2, ...
// with its own working tile, P tile and softmax state; all waves share the barriers, so the
// two teams advance in lockstep, each barrier covering two tiles. At the end the teams'
// (max, sum, O) are merged through LDS. Within a team, wave v (0..3) scores tile rows
// 16*(v>>1).. x heads 16*(v&1).. and accumulates O for channels 128v..128v+127.
template <bool FP8, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void sparse_mla_kernel(
    int W, int H, int B, int splits, int split_len, float sm_scale,
    const uint16_t *__restrict__ q_abs, const int32_t *__restrict__ token_ids,
    const int32_t *__restrict__ row_seq, const void *__restrict__ kv,
    const float *__restrict__ kv_scales, long long kv_rows, int S,
    const int32_t *__restrict__ block_table, int max_blocks, int block_size,
    float *__restrict__ out, float *__restrict__ lse, float *__restrict__ ws) {
    // fp8: a private raw ring per wave (2 stages x 8 rows) + one working tile per team.
    // bf16: a ring of 2 working tiles per team.
    constexpr int kRingBytes = FP8 ? (8 * 2 * kRawWave + 2 * kWorkTile) : 4 * kWorkTile;
    constexpr int kRowBytes = FP8 ? kRawRow : kWorkRow;   // bytes a fetched row takes
    constexpr int kRowsPerLoad = 1024 / kRowBytes;         // rows per 64-lane 16-byte load
    constexpr int kLoadsPerWave = 8 / kRowsPerLoad;        // per wave per tile
    constexpr int kLanesPerRow = kWave / kRowsPerLoad;
    static_assert(kRingBytes >= 2 * 32 * kC * 4 / 2, "merge area fits in the ring");

    __shared__ __attribute__((aligned(16))) uint8_t ring[kRingBytes];
    __shared__ __attribute__((aligned(16))) uint16_t pl[2][32 * kPStride];
    __shared__ int rows_s[kMaxSplit];
    __shared__ float scale_s[kMaxSplit];
    __shared__ float red[8][16];
    __shared__ float alpha_s[2][32];
    __shared__ float msum_s[2][32];
    __shared__ float lsum_s[2][32];
    __shared__ int last_s;
    __shared__ int rescale_s[2][2];

    const int r = blockIdx.x;
    const int split = blockIdx.y;
    const int g = blockIdx.z;
    const int G = gridDim.z;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;       // 0..7
    const int tm = wave >> 2;           // team
    const int v = wave & 3;             // wave within the team
    const int b = row_seq[r];
    const bool row_ok = b >= 0 && b < B;
    const int s0 = split * split_len;
    const int n_slots = max(0, min(split_len, W - s0));
    const uint8_t *kvb = static_cast<const uint8_t *>(kv);

    // Query fragment for S^T = K Q^T (B operand): head column lane&15 of this wave's 16,
    // channels 32*st + (lane>>4)*8 .. +8 at step st. Issued first; used after the prologue.
    const int qk_head_local = 16 * (v & 1) + (lane & 15);
    const int qk_head = g * 32 + qk_head_local;
    u32x4 qf[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) {
        qf[st] = u32x4{0u, 0u, 0u, 0u};
        if (qk_head < H)
            qf[st] = *reinterpret_cast<const u32x4 *>(q_abs + ((size_t)r * H + qk_head) * kC +
                                                      32 * st + (lane >> 4) * 8);
    }

    // ---- prologue: resolve every slot of the split to a latent row (or -1) and its scale
    if (tid == 0) last_s = -1;
    if (tid < 4) rescale_s[tid >> 1][tid & 1] = 0;
    __syncthreads();
    int my_last = -1;
    for (int i = tid; i < n_slots; i += kThreads) {
        const int tok = token_ids[(size_t)r * W + s0 + i];
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
        float sc = 1.0f;
        if constexpr (FP8) sc = row >= 0 ? kv_scales[row] : 0.0f;
        rows_s[i] = (int)row;
        scale_s[i] = sc;
        if (row >= 0) my_last = i;
    }
    if (my_last >= 0) atomicMax(&last_s, my_last);
    wait_vm<0>();  // the query fragment is in registers before any tile load is issued
    __syncthreads();
    const int n_tiles = (last_s + kTile) / kTile;  // through the last slot with a token
    const int n_iter = (n_tiles + 1) / 2;           // tile pairs

    // ---- LDS addressing, hoisted out of the tile loop (all offsets are per lane).
    uint8_t *const work0 = FP8 ? ring + 8 * 2 * kRawWave + tm * kWorkTile : ring + 2 * tm * kWorkTile;
    // fetch: wave v fetches rows 8v..8v+7 of its team's tiles; a slot without a token fetches
    // latent row 0 (finite data; its weight is zero). fp8 rows go to the wave's own raw ring.
    auto stage_of = [&](int t) -> uint8_t * {   // where tile t's fetched rows of this wave go
        const int st2 = (t >> 1) & 1;
        if constexpr (FP8) return ring + (wave * 2 + st2) * kRawWave;
        else return ring + (2 * tm + st2) * kWorkTile + 8 * v * kWorkRow;
    };
    auto issue = [&](int t) {
        uint8_t *stage = stage_of(t);
#pragma unroll
        for (int k = 0; k < kLoadsPerWave; ++k) {
            const int rl = k * kRowsPerLoad + lane / kLanesPerRow;  // row within the wave's 8
            const int rr = 8 * v + rl;                              // row within the tile
            const int pos = lane % kLanesPerRow;
            const int slot = t * kTile + rr;
            int prow = slot < n_slots ? rows_s[slot] : -1;
            if (prow < 0) prow = 0;
            const int chunk = FP8 ? (pos ^ (8 * (rr & 1))) : (pos ^ swz_work(rr));
            const uint8_t *src = kvb + (size_t)prow * kRowBytes + 16 * chunk;
            dma16(src, __builtin_amdgcn_readfirstlane(
                           lds_offset(stage + k * kRowsPerLoad * kRowBytes)));
        }
    };
    // fp8 conversion: lane -> row 8v + lane/8, raw chunks (lane&7) + 8k, k = 0..3.
    const int cv_row = 8 * v + (lane >> 3);
    const uint32_t cv_raw = (uint32_t)((lane >> 3) * kRawRow + 16 * (lane & 7));
    const int cv_flip = 8 * (cv_row & 1) * 16;  // raw chunk c sits at c ^ 8(r&1): 128-byte swap
    const int cv_sw = swz_work(cv_row);
    const uint32_t cv_w0 = (uint32_t)(cv_row * kWorkRow + 16 * ((2 * (lane & 7)) ^ cv_sw));
    const uint32_t cv_w1 = (uint32_t)(cv_row * kWorkRow + 16 * ((2 * (lane & 7) + 1) ^ cv_sw));
    // QK operand: row tb + (lane&15), chunk 4*st + (lane>>4) at position ^ swz_work(row):
    // offset = row*1024 + 64*(st ^ kq) + 16*lq with kq, lq from the row's swizzle.
    const int tb = 16 * (v >> 1);
    const int qk_row = tb + (lane & 15);
    const int qk_sw = swz_work(qk_row);
    const uint32_t qk_base = (uint32_t)(qk_row * kWorkRow + 16 * (((lane >> 4) ^ qk_sw) & 3));
    const int qk_k = qk_sw >> 2;
    uint32_t qk_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qk_off[j] = qk_base + 64 * (j ^ qk_k);
    // V operand (two transpose reads per fragment): source lane src of 16-lane group grp reads
    // row 16*ks + 8*(grp>>1) + (src>>2) (+4), 4 channels at 128v + 32nt + 16(grp&1) + 4(src&3).
    const int grp = lane >> 4, src = lane & 15;
    const int va = src >> 2;                    // row & 3, equal for both reads
    const int vb = 2 * (grp >> 1);              // (row >> 2) & 3 of the first read
    const int ve = 2 * (grp & 1) + ((src & 3) >> 1);
    uint32_t v_off[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            v_off[h][nt] = (uint32_t)((8 * (grp >> 1) + va + 4 * h) * kWorkRow + 256 * v +
                                      64 * (nt ^ va) + 16 * (ve ^ (vb + h)) + 8 * (src & 1));

    for (int t = tm; t < 2 && t < n_tiles; t += 2) issue(t);   // first tile of each team
    if constexpr (FP8) {
        if (tm + 2 < n_tiles) issue(tm + 2);                     // fp8: one more in flight
    }

    float m_ref = -INFINITY;  // reference maximum of head qk_head in this team
    float l_run = 0.0f;       // this lane's share of the running sum
    f32x16 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x16{};

    for (int it = 0; it < n_iter; ++it) {
        const int t = 2 * it + tm;          // this team's tile (may be past the end: idle)
        const bool live = t < n_tiles;
        const int par = it & 1;
        uint8_t *Wt;
        if constexpr (FP8) {
            // This wave's rows of tile t landed once at most one later tile of it is in flight.
            if (live) {
                if (t + 2 < n_tiles) wait_vm<kLoadsPerWave>();
                else wait_vm<0>();
            }
            Wt = work0;
            lds_barrier();  // A0: the team's previous tile is fully consumed
            if (live) {
                const uint8_t *R = stage_of(t);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const u32x4 raw = lds_load<u32x4>(R, cv_raw ^ (uint32_t)(cv_flip) ^ (uint32_t)(128 * k));
                    const u32x2 a0 = e4m3x4_to_bf16x4(raw.x), a1 = e4m3x4_to_bf16x4(raw.y);
                    const u32x2 a2 = e4m3x4_to_bf16x4(raw.z), a3 = e4m3x4_to_bf16x4(raw.w);
                    *reinterpret_cast<u32x4 *>(Wt + cv_w0 + 256 * k) = u32x4{a0.x, a0.y, a1.x, a1.y};
                    *reinterpret_cast<u32x4 *>(Wt + cv_w1 + 256 * k) = u32x4{a2.x, a2.y, a3.x, a3.y};
                }
                if (t + 4 < n_tiles) issue(t + 4);  // refills the raw stage just converted
            }
        } else {
            if (live) wait_vm<0>();
            Wt = ring + (2 * tm + ((t >> 1) & 1)) * kWorkTile;
        }
        lds_barrier();  // A: working tiles complete; tile t-2 of the team fully consumed
        if constexpr (!FP8) {
            // bf16 rows land directly in working tiles read by the whole team, so the stage
            // of tile t-2 is refilled only after barrier A.
            if (live && t + 2 < n_tiles) issue(t + 2);
        }

        // ---- logits S^T[token][head] for this wave's 16 tokens x 16 heads (two chains)
        float x[4], sc[4];
        float tmax = -INFINITY;
        if (live) {
            f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 16; st += 2) {
                const u32x4 a0 = lds_load<u32x4>(Wt, qk_off[st & 3] + 256 * (st >> 2));
                const u32x4 a1 = lds_load<u32x4>(Wt, qk_off[(st + 1) & 3] + 256 * ((st + 1) >> 2));
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qf[st]), sa, 0, 0, 0);
                sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qf[st + 1]), sb, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int slot = t * kTile + tb + (lane >> 4) * 4 + i;
                const bool ok = slot < n_slots && rows_s[slot] >= 0;
                sc[i] = ok ? scale_s[slot] : 0.0f;
                x[i] = ok ? (sa[i] + sb[i]) * (sm_scale * sc[i]) : -INFINITY;
                tmax = fmaxf(tmax, x[i]);
            }
            tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
            tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
            if (lane < 16) red[wave][lane] = tmax;
        }
        lds_barrier();  // B: tile maxima

        uint16_t *P = pl[tm];
        if (live) {
            const float m_tile = fmaxf(red[wave][lane & 15], red[wave ^ 2][lane & 15]);
            float alpha = 1.0f;
            if (m_tile > m_ref + kRescaleSlack) {  // also true for the first tile with a token
                alpha = m_ref == -INFINITY ? 0.0f : fast_exp(m_ref - m_tile);
                m_ref = m_tile;
            }
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = x[i] == -INFINITY ? 0.0f : fast_exp(x[i] - m_ref);
            l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
            *reinterpret_cast<u32x2 *>(P + qk_head_local * kPStride + tb + (lane >> 4) * 4) =
                u32x2{pack_bf16x2(p[0] * sc[0], p[1] * sc[1]), pack_bf16x2(p[2] * sc[2], p[3] * sc[3])};
            if ((v >> 1) == 0 && lane < 16) {
                alpha_s[tm][qk_head_local] = alpha;
                if (alpha != 1.0f) rescale_s[tm][par] = 1;
            }
        }
        if (v == 0 && lane == 0) rescale_s[tm][par ^ 1] = 0;  // read only after the next barrier C
        lds_barrier();  // C: P, alpha and the rescale flag visible

        // ---- O[head][channel] += P . V over the tile's 32 tokens; this wave: 128 channels.
        // V fragments come from the working tile with the LDS transpose read: in each 16-lane
        // group the result lane holds one channel down 4 consecutive tokens; two reads give 8.
        if (live) {
            if (rescale_s[tm][par]) {
                float al[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) al[i] = alpha_s[tm][8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[nt][i] *= al[i];
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(P + (lane & 31) * kPStride + 16 * ks +
                                                                 (lane >> 5) * 8);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t *>(
                        Wt + v_off[0][nt] + 16 * kWorkRow * ks));
                    const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t *>(
                        Wt + v_off[1][nt] + 16 * kWorkRow * ks));
                    const u32x4 vv = {lo.x, lo.y, hi.x, hi.y};
                    acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(vv),
                                                                      acc[nt], 0, 0, 0);
                }
            }
        }
        // The next pair's first barrier orders these reads before the tiles are reused.
    }

    // ---- finish: per-head sums of each team, then the two teams are merged
    l_run += shfl_xor_f(l_run, 16);
    l_run += shfl_xor_f(l_run, 32);
    __syncthreads();
    if (lane < 16) red[wave][lane] = l_run;
    __syncthreads();
    if (v < 2 && lane < 16) {
        lsum_s[tm][qk_head_local] = red[wave][lane] + red[wave ^ 2][lane];
        msum_s[tm][qk_head_local] = m_ref;
    }
    __syncthreads();
    // Team weights per accumulator row (head) m: exp(m_team - M), M the larger maximum.
    float wt[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float m0 = msum_s[0][m], m1 = msum_s[1][m];
        const float M = fmaxf(m0, m1);
        const float mine = tm == 0 ? m0 : m1;
        wt[i] = mine == -INFINITY ? 0.0f : fast_exp(mine - M);
    }
    float *xch = reinterpret_cast<float *>(ring);  // team 1's weighted O, [32 heads][512]
    if (tm == 1) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int ch = 128 * v + 32 * nt + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                xch[m * kC + ch] = acc[nt][i] * wt[i];
            }
        }
    }
    __syncthreads();
    if (tm == 1) return;

    float Ls[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float m0 = msum_s[0][m], m1 = msum_s[1][m];
        const float M = fmaxf(m0, m1);
        const float w0 = m0 == -INFINITY ? 0.0f : fast_exp(m0 - M);
        const float w1 = m1 == -INFINITY ? 0.0f : fast_exp(m1 - M);
        Ls[i] = lsum_s[0][m] * w0 + lsum_s[1][m] * w1;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int ch = 128 * v + 32 * nt + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            acc[nt][i] = acc[nt][i] * wt[i] + xch[m * kC + ch];
        }
    }

    if (splits == 1) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int ch = 128 * v + 32 * nt + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                const int hg = g * 32 + m;
                if (hg < H) out[((size_t)r * H + hg) * kC + ch] = Ls[i] > 0.0f ? acc[nt][i] / Ls[i] : 0.0f;
            }
        }
        if (lse != nullptr && tid < 32 && g * 32 + tid < H) {
            const float M = fmaxf(msum_s[0][tid], msum_s[1][tid]);
            const float w0 = msum_s[0][tid] == -INFINITY ? 0.0f : fast_exp(msum_s[0][tid] - M);
            const float w1 = msum_s[1][tid] == -INFINITY ? 0.0f : fast_exp(msum_s[1][tid] - M);
            const float L = lsum_s[0][tid] * w0 + lsum_s[1][tid] * w1;
            lse[(size_t)r * H + g * 32 + tid] = L > 0.0f ? M + logf(L) : -INFINITY;
        }
    } else {
        float *part = ws + (((size_t)r * G + g) * splits + split) * kPartFloats;
        if (tid < 32) {
            const float M = fmaxf(msum_s[0][tid], msum_s[1][tid]);
            const float w0 = msum_s[0][tid] == -INFINITY ? 0.0f : fast_exp(msum_s[0][tid] - M);
            const float w1 = msum_s[1][tid] == -INFINITY ? 0.0f : fast_exp(msum_s[1][tid] - M);
            part[tid] = M;
            part[32 + tid] = lsum_s[0][tid] * w0 + lsum_s[1][tid] * w1;
        }
        if (n_tiles > 0) {  // a split without tokens leaves O unwritten; its sum is 0
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int ch = 128 * v + 32 * nt + (lane & 31);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    part[64 + m * kC + ch] = acc[nt][i];
                }
            }
        }
    }
}

// Merge the per-split partial results of one (row, head): log-sum-exp weights. One block
// of 128 threads per (row, head); each thread owns 4 channels.
__global__ __launch_bounds__(128) void mla_combine_kernel(int H, int splits,
                                                          const float *__restrict__ ws,
                                                          float *__restrict__ out,
                                                          float *__restrict__ lse) {
    __shared__ float wgt[kMaxSplits];
    __shared__ float norm_s[2];
    const int r = blockIdx.x;
    const int h = blockIdx.y;
    const int G = (H + 31) / 32;
    const int g = h >> 5, m = h & 31;
    const int tid = threadIdx.x;
    const float *base = ws + ((size_t)r * G + g) * splits * kPartFloats;
    if (tid < kWave) {
        // splits <= 64: one lane per split
        const float ms = tid < splits ? base[(size_t)tid * kPartFloats + m] : -INFINITY;
        const float ls = tid < splits ? base[(size_t)tid * kPartFloats + 32 + m] : 0.0f;
        float M = ms;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) M = fmaxf(M, shfl_xor_f(M, d));
        const float wv = (ls > 0.0f && M != -INFINITY) ? fast_exp(ms - M) : 0.0f;
        float L = ls * wv;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) L += shfl_xor_f(L, d);
        if (tid < splits) wgt[tid] = wv;
        if (tid == 0) {
            norm_s[0] = L;
            norm_s[1] = M;
        }
    }
    __syncthreads();
    const float L = norm_s[0];
    const int c = tid * 4;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
        const float wv = wgt[s];
        if (wv == 0.0f) continue;  // no token in that split: its O was not written
        const f32x4 v = *reinterpret_cast<const f32x4 *>(base + (size_t)s * kPartFloats + 64 +
                                                         m * kC + c);
        o += v * wv;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    *reinterpret_cast<f32x4 *>(out + ((size_t)r * H + h) * kC + c) = o * inv;
    if (lse != nullptr && tid == 0) lse[(size_t)r * H + h] = L > 0.0f ? norm_s[1] + logf(L) : -INFINITY;
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
    hipLaunchKernelGGL(mla_combine_kernel, dim3(Q, H), dim3(128), 0, stream, H, plan.splits,
                       static_cast<const float *>(ws), out, lse);
    return hipGetLastError();
}

}  // namespace

// Split the token slots so that about 256 blocks (one 8-wave block per compute unit) run,
// with at least 64 slots per split, at most kMaxSplit slots per split and at most
// kMaxSplits splits; a row that already gives enough blocks is not split.
MlaPlan plan_sparse_mla(int Q, int W, int H) {
    MlaPlan p;
    p.groups = (H + 31) / 32;
    const long long wr = ((long long)W + kTile - 1) / kTile * kTile;
    const long long work = (long long)W * Q * p.groups;
    long long per = (work + 255) / 256;
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

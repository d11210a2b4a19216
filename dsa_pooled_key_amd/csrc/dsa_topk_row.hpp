// dsa_topk_row.hpp -- selection of one row's best pools and, optionally, their token ids,
// by a 1024-thread block whose threads hold the row's keys in registers.
//
// mod.rs, "Shape of the pipeline": [Q, P] scores -> [Q, select_k] pool ids; the token-id
// expansion follows the same page ("Checkpoint and kernel facts": every slot written, -1 for
// none). The ranking key is (score descending, pool index ascending) and the chosen ids are
// written in ascending order, so the result is unique.
//
// Thread t holds the order-preserving 32-bit keys of pools [t*KPT, t*KPT + KPT) (key 0 marks a
// non-candidate; every candidate maps above it). When there are more candidates than Kw, the
// candidates' smallest and largest scores set 2048 equal-width value bins; an LDS histogram and
// a one-wave scan find the bin holding the Kw-th largest key; one wave ranks that bin's keys
// exactly (larger bins, e.g. many equal scores, use 8-bit radix passes). Every key above the
// cutoff is taken, plus the lowest-index keys equal to it (an exclusive prefix count of equal
// keys in pool order), and a block prefix sum of per-thread counts places the ids in ascending
// order. Wave reductions and scans run on DPP and lane reads.
#pragma once

#include "dsa_device.hpp"
#include "dsa_phase.hpp"

namespace dsa {
namespace topk {

constexpr int kThreads = 1024;
constexpr int kBins = 2 * kThreads;  // value bins of the first stage

// Token-id expansion of a selection (the expand_selection step), fused into the top-k block.
struct ExpandArgs {
    int KP, topk, W, tail, B, S, first_key;
    int vec8;  // KP = 8, W % 4 == 0 and token_ids 16-byte aligned: a pool's slots are two int4
    const int32_t *row_seq;
    const int32_t *row_pos;
    const uint8_t *valid;
    int32_t *token_ids;
};


constexpr int kMaxMembers = kWave;  // cutoff bins up to this size are ranked by one wave
// Selections up to this width are staged in LDS and written (with their token ids) by
// consecutive threads, one pool each; wider ones are written by the selecting threads.
constexpr int kStageSel = 2048;

// LDS of one row's selection.
struct Smem {
    int scratch[kThreads / kWave + 1];
    uint32_t red3[3][kThreads / kWave];
    uint32_t hist[256];
    __attribute__((aligned(16))) uint32_t bins[kBins];
    uint32_t mem[kMaxMembers];
    int sel_s[kStageSel];
    int n_mem;
    uint32_t pick[3];
};

// Thread t's keys of row srow/crow: pools [t*KPT, t*KPT + KPT), key 0 where cand is 0 or the
// pool is past P. vec: P and both row bases allow 16-byte loads (scores) and 16- or 4-byte
// loads (cand).
template <int KPT>
__device__ __forceinline__ void load_keys(int P, int vec, const float *__restrict__ srow,
                                          const uint8_t *__restrict__ crow, uint32_t (&key)[KPT]) {
    const int base = threadIdx.x * KPT;
    if (KPT >= 16 && vec && base + KPT <= P) {
#pragma unroll
        for (int i = 0; i < KPT; i += 16) {
            const u32x4 cv = *reinterpret_cast<const u32x4 *>(crow + base + i);
            const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 sv = *reinterpret_cast<const f32x4 *>(srow + base + i + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    key[i + 4 * q + e] = ((cw[q] >> (8 * e)) & 0xffu) ? ordered_key(sv[e]) : 0u;
            }
        }
    } else if (KPT >= 4 && vec && base + KPT <= P) {
#pragma unroll
        for (int i = 0; i < KPT; i += 4) {
            const f32x4 sv = *reinterpret_cast<const f32x4 *>(srow + base + i);
            const uint32_t cv = *reinterpret_cast<const uint32_t *>(crow + base + i);
#pragma unroll
            for (int e = 0; e < 4 && i + e < KPT; ++e)
                key[i + e] = ((cv >> (8 * e)) & 0xffu) ? ordered_key(sv[e]) : 0u;
        }
    } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int p = base + i;
            key[i] = (p < P && crow[p]) ? ordered_key(srow[p]) : 0u;
        }
    }
}

// Row r's selection from its keys (thread t: key slots t*KPT ..). Writes sel[r, 0..Kw) and,
// with EXPAND, token_ids[r, 0..W). Key slot i stands for pool pool0 + i, or for pool ids[i]
// when an id table (LDS, ascending over the slots that hold candidates) is given; ties go to
// the lower slot either way. Called by all kThreads threads of the block.
template <int KPT, bool EXPAND, bool KEEP_BINS = (KPT <= 16)>
__device__ __forceinline__ void select_row(int r, int P, int Kw, uint32_t (&key)[KPT],
                                           int32_t *__restrict__ sel, const ExpandArgs &ex,
                                           Smem &sm, int pool0 = 0,
                                           const int *ids = nullptr) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int base = tid * KPT;
    int *const scratch = sm.scratch;
    uint32_t (&red3)[3][kThreads / kWave] = sm.red3;
    uint32_t *const hist = sm.hist;
    uint32_t *const bins = sm.bins;
    uint32_t *const mem = sm.mem;
    int &n_mem = sm.n_mem;
    uint32_t *const pick = sm.pick;
    // Candidate count and the largest and smallest candidate key, in one block reduction.
    uint32_t nc = 0u, kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        nc += key[i] != 0u;
        kmax = key[i] > kmax ? key[i] : kmax;
        if (key[i] != 0u) kmin = key[i] < kmin ? key[i] : kmin;
    }
    nc = wave_sum_u32(nc);  // unsigned comparisons throughout
    kmax = wave_max_u32(kmax);
    kmin = wave_min_u32(kmin);
    if (lane == 0) {
        red3[0][wave] = nc;
        red3[1][wave] = kmax;
        red3[2][wave] = kmin;
    }
    DSA_PHASE(1, 1);  // keys loaded and reduced in the wave
    if (tid == 0) n_mem = 0;
    for (int i = tid; i < kBins; i += kThreads) bins[i] = 0u;  // used only past this barrier
    __syncthreads();
    int n_cand = 0;
    kmax = 0u;
    kmin = 0xffffffffu;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
        n_cand += (int)red3[0][w];
        kmax = red3[1][w] > kmax ? red3[1][w] : kmax;
        kmin = red3[2][w] < kmin ? red3[2][w] : kmin;
    }
    DSA_PHASE(1, 2);  // block reduction done
    const int take = n_cand < Kw ? n_cand : Kw;

    uint32_t thr = 0u;  // take every key > thr, plus `need` of the keys == thr
    int need = 0;
    int eq_all = n_cand > Kw ? -1 : 0;  // keys == thr when known (then no tie scan is needed)
    if (n_cand > Kw) {
        // Stage 1: bucket the candidates by value into kBins equal-width bins between the
        // smallest and largest score (the bin index never decreases as the score grows), and
        // find the bin b* holding the Kw-th largest; every key in a higher bin is larger than
        // every key in b*, every key in a lower one smaller. A span that is zero or not
        // representable puts everything in bin 0.
        const float smax = ordered_key_value(kmax), smin = ordered_key_value(kmin);
        float inv = (float)kBins / (smax - smin);
        if (!(inv < 3.0e38f)) inv = 0.0f;  // also catches NaN
        auto bin_of = [&](uint32_t key) {
            const int bn = (int)((ordered_key_value(key) - smin) * inv);
            return bn < 0 ? 0 : (bn >= kBins ? kBins - 1 : bn);
        };
        // With KEEP_BINS the bins stay in registers for the membership test below; otherwise
        // they are computed again there (fewer registers).
        constexpr bool kKeepBins = KEEP_BINS;
        int bn[kKeepBins ? KPT : 1];
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int bi = key[i] != 0u ? bin_of(key[i]) : -1;
            if constexpr (kKeepBins) bn[i] = bi;
            if (bi >= 0) atomicAdd(&bins[bi], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // Wave 0 scans the bins from the top: lane l holds bins kBins-1-32l down to
            // kBins-32-32l, a wave prefix sum finds the lane, the lane walks its 32 bins.
            constexpr int kPerLane = kBins / kWave;
            const int top = kBins - 1 - kPerLane * tid;
            uint32_t cnt[kPerLane];
#pragma unroll
            for (int q = 0; q < kPerLane; q += 4) {
                const u32x4 v4 = *reinterpret_cast<const u32x4 *>(&bins[top - q - 3]);
                cnt[q] = v4.w;
                cnt[q + 1] = v4.z;
                cnt[q + 2] = v4.y;
                cnt[q + 3] = v4.x;
            }
            uint32_t sum = 0u;
#pragma unroll
            for (int q = 0; q < kPerLane; ++q) sum += cnt[q];
            const uint32_t inc = wave_incl_sum(sum);
            uint32_t above = inc - sum;
            const uint32_t kk = (uint32_t)Kw;
            if (above < kk && kk <= inc) {
                int q = 0;
                while (kk > above + cnt[q]) above += cnt[q++];
                pick[0] = (uint32_t)(top - q);
                pick[1] = above;
                pick[2] = cnt[q];
            }
        }
        __syncthreads();
        DSA_PHASE(1, 3);  // histogram scanned, cutoff bin known
        const int bstar = (int)pick[0];
        int k = Kw - (int)pick[1];  // rank of the cutoff inside b*
        const int members = (int)pick[2];
        static_assert(KPT <= 64, "membership mask");
        uint64_t member = 0u;  // keys of this thread that fall in b*
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            if ((kKeepBins ? bn[kKeepBins ? i : 0] : (key[i] != 0u ? bin_of(key[i]) : -1)) == bstar)
                member |= 1ull << i;
        // pick is rewritten only after the next barrier, which every thread reaches after
        // reading it above.
        if (members <= kMaxMembers) {
            // Stage 2 (small bin): gather its keys and let one wave rank them exactly.
#pragma unroll
            for (int i = 0; i < KPT; ++i)
                if ((member >> i) & 1ull) mem[atomicAdd(&n_mem, 1)] = key[i];
            __syncthreads();
            if (tid < kWave) {
                const uint32_t m = tid < members ? mem[tid] : 0u;
                int gt = 0, eq = 0;
                for (int j = 0; j < members; ++j) {  // lane j's key, broadcast from a register
                    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)m, j);
                    gt += o > m;
                    eq += o == m;
                }
                if (tid < members && gt < k && k <= gt + eq) {  // equal keys write equal values
                    pick[0] = m;
                    pick[1] = (uint32_t)(k - gt);
                    pick[2] = (uint32_t)eq;
                }
            }
            __syncthreads();
            thr = pick[0];
            need = (int)pick[1];
            eq_all = (int)pick[2];
        } else {
            // Stage 2 (large bin, e.g. many equal scores): exact most-significant-digit radix
            // select of the k-th largest key among the members of b* (8-bit LDS histograms).
            uint32_t prefix = 0u, pmask = 0u;
            for (int shift = 24; shift >= 0; shift -= 8) {
                if (tid < 256) hist[tid] = 0u;
                __syncthreads();
#pragma unroll
                for (int i = 0; i < KPT; ++i)
                    if (((member >> i) & 1ull) && (key[i] & pmask) == prefix)
                        atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
                __syncthreads();
                if (tid < kWave) {
                    // lane l covers digits 255-4l .. 252-4l, scanned from the top
                    const int d0 = 255 - 4 * tid;
                    const uint32_t c0 = hist[d0], c1 = hist[d0 - 1], c2 = hist[d0 - 2], c3 = hist[d0 - 3];
                    const uint32_t sm = c0 + c1 + c2 + c3;
                    const uint32_t inc = wave_incl_sum(sm);
                    const uint32_t abv = inc - sm;
                    const uint32_t kk = (uint32_t)k;
                    if (abv < kk && kk <= inc) {
                        uint32_t a = abv;
                        int digit = d0;
                        if (kk > a + c0) {
                            a += c0;
                            digit = d0 - 1;
                            if (kk > a + c1) {
                                a += c1;
                                digit = d0 - 2;
                                if (kk > a + c2) {
                                    a += c2;
                                    digit = d0 - 3;
                                }
                            }
                        }
                        pick[0] = (uint32_t)digit;
                        pick[1] = a;
                    }
                }
                __syncthreads();
                prefix |= pick[0] << shift;
                pmask |= 255u << shift;
                k -= (int)pick[1];
                __syncthreads();
            }
            thr = prefix;
            need = k;
        }
    }

    DSA_PHASE(1, 4);  // cutoff key known
    // Output positions in pool order: every key above thr, plus the first `need` keys equal to
    // it (the tie scan is skipped when all of them are taken).
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        gt += key[i] > thr;
        eq += key[i] == thr && key[i] != 0u;
    }
    int take_eq = eq;
    if (eq_all != need) {
        int eq_total;
        const int eq_before = block_exclusive_scan<kThreads>(eq, scratch, &eq_total);
        take_eq = need - eq_before;
        take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
    }
    int total;
    int o = block_exclusive_scan<kThreads>(gt + take_eq, scratch, &total);
    // Each thread writes the ids it selects at their output positions and, fused, the token
    // ids of those pools (slots o*KP .. o*KP+KP-1); positions run in pool order across the
    // block, so a wave's stores land on neighbouring addresses.
    int32_t *orow = sel + (size_t)r * Kw;
    int32_t *trow = EXPAND ? ex.token_ids + (size_t)r * ex.W : nullptr;
    // The keys this thread selects, as a bit mask: all above thr, then its first take_eq keys
    // equal to thr; the writes below visit only the set bits.
    uint64_t smask = 0u, emask = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (key[i] > thr) smask |= 1ull << i;
        if (key[i] == thr && key[i] != 0u) emask |= 1ull << i;
    }
    for (int k = 0; k < take_eq; ++k) {
        smask |= emask & (0ull - emask);
        emask &= emask - 1ull;
    }
    // Selected pool p at output position o: its id and, fused, its KP token ids.
    auto write_pool = [&](int o, int p) {
        orow[o] = p;
        if constexpr (EXPAND) {
            const int t0 = ex.first_key + p * ex.KP;
            int32_t *dst = trow + (size_t)o * ex.KP;
            if (ex.vec8) {  // KP = 8 and 16-byte aligned slots: two 16-byte stores
                reinterpret_cast<int4 *>(dst)[0] = int4{t0, t0 + 1, t0 + 2, t0 + 3};
                reinterpret_cast<int4 *>(dst)[1] = int4{t0 + 4, t0 + 5, t0 + 6, t0 + 7};
            } else {
                for (int t = 0; t < ex.KP; ++t) dst[t] = t0 + t;
            }
        }
    };
    DSA_PHASE(1, 5);  // output positions known
    auto pool_of = [&](int i) { return ids != nullptr ? ids[base + i] : pool0 + base + i; };
    if (Kw <= kStageSel) {
        // The ids go to LDS at their positions; after one barrier thread j writes position j,
        // so a row whose selection sits in few threads (a context of few pools) still spreads
        // its stores over the block, and ids and token ids go out in coalesced runs.
        while (smask != 0u && o < Kw) {
            sm.sel_s[o++] = pool_of(__builtin_ctzll(smask));
            smask &= smask - 1ull;
        }
        __syncthreads();
        for (int j = tid; j < Kw; j += kThreads) {
            if (j < take) write_pool(j, sm.sel_s[j]);
            else orow[j] = -1;
        }
    } else {
        while (smask != 0u && o < Kw) {
            write_pool(o, pool_of(__builtin_ctzll(smask)));
            smask &= smask - 1ull;
            ++o;
        }
        for (int i = take + tid; i < Kw; i += kThreads) orow[i] = -1;
    }
    DSA_PHASE(1, 6);  // selection written
    if constexpr (EXPAND) {
        // The remaining token slots (as expand_selection): -1 up to topk, then the tail tokens
        // after the last whole pool up to row_pos, each only if valid.
        const int b = ex.row_seq[r];
        const long long pos = ex.row_pos[r];
        const bool tail_ok = ex.tail && b >= 0 && b < ex.B && pos + 1 > ex.first_key;
        const long long start = ex.first_key + ((pos + 1 - ex.first_key) / ex.KP) * ex.KP;
        for (int i = take * ex.KP + tid; i < ex.W; i += kThreads) {
            int v = -1;
            if (i >= ex.topk && tail_ok) {
                const long long t = start + (i - ex.topk);
                if (t <= pos && t < ex.S && ex.valid[(size_t)b * ex.S + t]) v = (int)t;
            }
            trow[i] = v;
        }
    }
}

}  // namespace topk
}  // namespace dsa

// topk_pools.hip -- per-row selection of the best pools (and, fused, their token ids).
//
// mod.rs, "Shape of the pipeline": [Q, P] scores -> [Q, select_k] pool ids. The pages fix
// neither the tie rule nor the output order; tp.rs warns that ties at the cutoff are order
// sensitive. Here the ranking key is (score descending, pool index ascending) and the chosen
// ids are written in ascending order, so the result is unique. One 1024-thread block per row
// loads the row's keys and runs the selection of dsa_topk_row.hpp; the fused variant also
// writes the row's token ids exactly as expand_selection does, so the selection never goes
// back to memory to be read again.
#include <mutex>

#include "dsa_device.hpp"
#include "dsa_launch.hpp"
#include "dsa_phase.hpp"

DSA_PHASE_TABLE(topk)

#include "dsa_topk_row.hpp"

namespace dsa {
namespace {

using namespace topk;

// PAIR: the form for more rows than compute units, held to 64 registers (the keys' value bins
// are computed again for the membership test instead of kept), so that two 1024-thread blocks
// share a CU (71.7 against 91.6 us for the 2,048 rows of prefill_2048_64k). With fewer rows a
// block's latency is what counts, and the unconstrained form is faster (10.2 against 11.9 us
// for fp8_mixed_b32's 32 rows).
template <int KPT, bool EXPAND, bool PAIR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PAIR ? 8 : 1))) void topk_pools_kernel(
    int P, int Kw, int vec, const float *__restrict__ scores, const uint8_t *__restrict__ cand,
    int32_t *__restrict__ sel, ExpandArgs ex) {
    __shared__ Smem sm;
    const int r = blockIdx.x;

    DSA_PHASE(1, 0);  // block start
    uint32_t key[KPT];
    load_keys<KPT>(P, vec, scores + (size_t)r * P, cand + (size_t)r * P, key);
    select_row<KPT, EXPAND, !PAIR && KPT <= 16>(r, P, Kw, key, sel, ex, sm);
    DSA_PHASE(1, 7);  // stores issued
}

// Two stages for rows that are few and long, which a block each would leave most of the chip
// idle for: stage 1 splits every row into segments of kSegPools pools and selects each
// segment's best Kw exactly (block (r, s), the same selection); every pool of the row's best Kw
// is among its segment's best Kw. Stage 2 selects the row's best Kw from the segments' picks
// (their scores gathered again by id) and expands them. Segments are in pool order and each
// lists its picks ascending, so the slot order of stage 2 is pool order and ties keep
// going to the lower pool.
constexpr int kSegKpt = 8;
constexpr int kSegPools = kThreads * kSegKpt;

__global__ __launch_bounds__(kThreads) void topk_segment_kernel(int P, int Kw, int nseg, int vec,
                                                                const float *__restrict__ scores,
                                                                const uint8_t *__restrict__ cand,
                                                                int32_t *__restrict__ picks) {
    __shared__ Smem sm;
    const int r = blockIdx.x, sg = blockIdx.y;
    const int p0 = sg * kSegPools;
    const int n = min(kSegPools, P - p0);
    uint32_t key[kSegKpt];
    load_keys<kSegKpt>(n, vec, scores + (size_t)r * P + p0, cand + (size_t)r * P + p0, key);
    select_row<kSegKpt, false>(r * nseg + sg, n, Kw, key, picks, ExpandArgs{}, sm, p0);
}

template <int KPT, bool EXPAND>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(int P, int Kw, int n,
                                                              const float *__restrict__ scores,
                                                              const int32_t *__restrict__ picks,
                                                              int32_t *__restrict__ sel,
                                                              ExpandArgs ex) {
    __shared__ Smem sm;
    __shared__ int ids_s[kThreads * KPT];
    const int r = blockIdx.x;
    const int base = threadIdx.x * KPT;
    int id[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int e = base + i;
        const int v = e < n ? picks[(size_t)r * n + e] : -1;
        id[i] = v >= 0 && v < P ? v : -1;
        ids_s[e] = id[i];
    }
    uint32_t key[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) key[i] = id[i] >= 0 ? ordered_key(scores[(size_t)r * P + id[i]]) : 0u;
    select_row<KPT, EXPAND>(r, n, Kw, key, sel, ex, sm, 0, ids_s);
}

// Segments a row for the two-stage selection, or 0 for one block a row. Two stages pay for
// few rows of more than 16,384 pools (one block holds 32 or 64 keys a thread there);
// measured on 32 rows of 16,384 pools one block a row is faster (10.2 against 13.6 us).
int topk_segments(int Q, int P, int Kw) {
    const int nseg = (P + kSegPools - 1) / kSegPools;
    if (Q > 64 || P <= 16384 || nseg < 2 || 4 * Kw > kSegPools ||
        (long long)nseg * Kw > 8 * kThreads)
        return 0;
    return nseg;
}

template <int KPT>
hipError_t launch_kpt(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                      int32_t *sel, const ExpandArgs *ex, hipStream_t stream) {
    // 16-byte score loads need a 16-byte aligned row start; candidate flags are read 16 (or 4)
    // at a time.
    const int vec = (KPT >= 16 ? (P & 15) == 0 && (reinterpret_cast<uintptr_t>(cand) & 15) == 0
                                : (P & 3) == 0 && (reinterpret_cast<uintptr_t>(cand) & 3) == 0) &&
                    (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
    const ExpandArgs exa = ex ? *ex : ExpandArgs{};
    bool pair = false;
    if constexpr (KPT == 16) {  // the only width whose 64-register form does not spill
        int cus = 0;
        const hipError_t e = device_cu_count(&cus);
        if (e != hipSuccess) return e;
        pair = Q > cus;
    }
    if (ex && pair)
        hipLaunchKernelGGL((topk_pools_kernel<KPT, true, true>), dim3(Q), dim3(kThreads), 0, stream, P,
                           Kw, vec, scores, cand, sel, exa);
    else if (ex)
        hipLaunchKernelGGL((topk_pools_kernel<KPT, true, false>), dim3(Q), dim3(kThreads), 0, stream, P,
                           Kw, vec, scores, cand, sel, exa);
    else if (pair)
        hipLaunchKernelGGL((topk_pools_kernel<KPT, false, true>), dim3(Q), dim3(kThreads), 0, stream, P,
                           Kw, vec, scores, cand, sel, exa);
    else
        hipLaunchKernelGGL((topk_pools_kernel<KPT, false, false>), dim3(Q), dim3(kThreads), 0, stream, P,
                           Kw, vec, scores, cand, sel, exa);
    return hipGetLastError();
}

template <int KPT>
hipError_t launch_merge(int Q, int P, int Kw, int n, const float *scores, const int32_t *picks,
                        int32_t *sel, const ExpandArgs *ex, hipStream_t stream) {
    if (ex)
        hipLaunchKernelGGL((topk_merge_kernel<KPT, true>), dim3(Q), dim3(kThreads), 0, stream, P, Kw,
                           n, scores, picks, sel, *ex);
    else
        hipLaunchKernelGGL((topk_merge_kernel<KPT, false>), dim3(Q), dim3(kThreads), 0, stream, P, Kw,
                           n, scores, picks, sel, ExpandArgs{});
    return hipGetLastError();
}

hipError_t launch_two_stage(int Q, int P, int Kw, int nseg, const float *scores,
                            const uint8_t *cand, int32_t *sel, const ExpandArgs *ex, void *ws,
                            hipStream_t stream) {
    int32_t *picks = static_cast<int32_t *>(ws);
    const int vec = (kSegPools & 15) == 0 && (P & 15) == 0 && (reinterpret_cast<uintptr_t>(cand) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
    hipLaunchKernelGGL(topk_segment_kernel, dim3(Q, nseg), dim3(kThreads), 0, stream, P, Kw, nseg, vec,
                       scores, cand, picks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n = nseg * Kw;
    if (n <= kThreads * 2) return launch_merge<2>(Q, P, Kw, n, scores, picks, sel, ex, stream);
    if (n <= kThreads * 4) return launch_merge<4>(Q, P, Kw, n, scores, picks, sel, ex, stream);
    return launch_merge<8>(Q, P, Kw, n, scores, picks, sel, ex, stream);
}

hipError_t launch_any(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                      int32_t *sel, const ExpandArgs *ex, void *ws, size_t ws_bytes,
                      hipStream_t stream) {
    if (Q == 0 || Kw == 0) return hipSuccess;
    const int nseg = topk_segments(Q, P, Kw);
    if (nseg > 0 && ws != nullptr && ws_bytes >= topk_workspace_bytes(Q, P, Kw))
        return launch_two_stage(Q, P, Kw, nseg, scores, cand, sel, ex, ws, stream);
    if (P <= kThreads * 1) return launch_kpt<1>(Q, P, Kw, scores, cand, sel, ex, stream);
    if (P <= kThreads * 2) return launch_kpt<2>(Q, P, Kw, scores, cand, sel, ex, stream);
    if (P <= kThreads * 4) return launch_kpt<4>(Q, P, Kw, scores, cand, sel, ex, stream);
    if (P <= kThreads * 8) return launch_kpt<8>(Q, P, Kw, scores, cand, sel, ex, stream);
    if (P <= kThreads * 16) return launch_kpt<16>(Q, P, Kw, scores, cand, sel, ex, stream);
    if (P <= kThreads * 32) return launch_kpt<32>(Q, P, Kw, scores, cand, sel, ex, stream);
    if (P <= kThreads * 64) return launch_kpt<64>(Q, P, Kw, scores, cand, sel, ex, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t device_cu_count(int *cus) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int count[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (count[dev] == 0) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        count[dev] = n > 0 ? n : 1;
    }
    *cus = count[dev];
    return hipSuccess;
}

size_t topk_workspace_bytes(int Q, int P, int Kw) {
    const int nseg = topk_segments(Q, P, Kw);
    return nseg > 0 ? (size_t)Q * nseg * Kw * sizeof(int32_t) : 0;
}

hipError_t launch_topk_pools(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                             int32_t *sel, void *ws, size_t ws_bytes, hipStream_t stream) {
    return launch_any(Q, P, Kw, scores, cand, sel, nullptr, ws, ws_bytes, stream);
}

hipError_t launch_topk_expand(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                              int32_t *sel, int KP, int topk, int W, bool tail, int B, int S,
                              int first_key, const int32_t *row_seq, const int32_t *row_pos,
                              const uint8_t *valid, int32_t *token_ids, void *ws,
                              size_t ws_bytes, hipStream_t stream) {
    if (Q == 0 || W == 0) return hipSuccess;
    if (Kw == 0)  // nothing to select: the plain expansion writes the -1 row and the tail
        return launch_expand_selection(Q, 0, KP, topk, W, tail, B, S, first_key, P, sel, row_seq,
                                       row_pos, valid, token_ids, stream);
    const int vec8 = KP == 8 && (W & 3) == 0 && (reinterpret_cast<uintptr_t>(token_ids) & 15) == 0;
    const ExpandArgs ex{KP, topk, W, tail ? 1 : 0, B, S, first_key, vec8, row_seq, row_pos, valid,
                        token_ids};
    return launch_any(Q, P, Kw, scores, cand, sel, &ex, ws, ws_bytes, stream);
}

}  // namespace dsa

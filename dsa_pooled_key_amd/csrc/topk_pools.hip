// topk_pools.hip -- per-row selection of the best pools (and, fused, their token ids).
//
// mod.rs, "Shape of the pipeline": [Q, P] scores -> [Q, select_k] pool ids. The pages fix
// neither the tie rule nor the output order; tp.rs warns that ties at the cutoff are order
// sensitive. Here the ranking key is (score descending, pool index ascending) and the chosen
// ids are written in ascending order, so the result is unique. One 1024-thread block per row
// loads the row's keys and runs the selection of dsa_topk_row.hpp; the fused variant also
// writes the row's token ids exactly as expand_selection does, so the selection never goes
// back to memory to be read again.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"
#include "dsa_topk_row.hpp"

namespace dsa {
namespace {

using namespace topk;

template <int KPT, bool EXPAND>
__global__ __launch_bounds__(kThreads) void topk_pools_kernel(int P, int Kw, int vec,
                                                              const float *__restrict__ scores,
                                                              const uint8_t *__restrict__ cand,
                                                              int32_t *__restrict__ sel,
                                                              ExpandArgs ex) {
    __shared__ Smem sm;
    const int r = blockIdx.x;
    const int tid = threadIdx.x;

    uint32_t key[KPT];
    load_keys<KPT>(P, vec, scores + (size_t)r * P, cand + (size_t)r * P, key);
    select_row<KPT, EXPAND>(r, P, Kw, key, sel, ex, sm);
}

template <int KPT>
hipError_t launch_kpt(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                      int32_t *sel, const ExpandArgs *ex, hipStream_t stream) {
    // 16-byte score loads need a 16-byte aligned row start; candidate flags are read 16 (or 4)
    // at a time.
    const int vec = (KPT >= 16 ? (P & 15) == 0 && (reinterpret_cast<uintptr_t>(cand) & 15) == 0
                                : (P & 3) == 0 && (reinterpret_cast<uintptr_t>(cand) & 3) == 0) &&
                    (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
    if (ex)
        hipLaunchKernelGGL((topk_pools_kernel<KPT, true>), dim3(Q), dim3(kThreads), 0, stream, P,
                           Kw, vec, scores, cand, sel, *ex);
    else
        hipLaunchKernelGGL((topk_pools_kernel<KPT, false>), dim3(Q), dim3(kThreads), 0, stream, P,
                           Kw, vec, scores, cand, sel, ExpandArgs{});
    return hipGetLastError();
}

hipError_t launch_any(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                      int32_t *sel, const ExpandArgs *ex, hipStream_t stream) {
    if (Q == 0 || Kw == 0) return hipSuccess;
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

hipError_t launch_topk_pools(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                             int32_t *sel, hipStream_t stream) {
    return launch_any(Q, P, Kw, scores, cand, sel, nullptr, stream);
}

hipError_t launch_topk_expand(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                              int32_t *sel, int KP, int topk, int W, bool tail, int B, int S,
                              int first_key, const int32_t *row_seq, const int32_t *row_pos,
                              const uint8_t *valid, int32_t *token_ids, hipStream_t stream) {
    if (Q == 0 || W == 0) return hipSuccess;
    if (Kw == 0)  // nothing to select: the plain expansion writes the -1 row and the tail
        return launch_expand_selection(Q, 0, KP, topk, W, tail, B, S, first_key, P, sel, row_seq,
                                       row_pos, valid, token_ids, stream);
    const int vec8 = KP == 8 && (W & 3) == 0 && (reinterpret_cast<uintptr_t>(token_ids) & 15) == 0;
    const ExpandArgs ex{KP, topk, W, tail ? 1 : 0, B, S, first_key, vec8, row_seq, row_pos, valid,
                        token_ids};
    return launch_any(Q, P, Kw, scores, cand, sel, &ex, stream);
}

}  // namespace dsa

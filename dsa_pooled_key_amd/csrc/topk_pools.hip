// topk_pools.hip -- per-row selection of the best pools.
//
// mod.rs, "Shape of the pipeline": [Q, P] scores -> [Q, select_k] pool ids. The pages fix
// neither the tie rule nor the output order; tp.rs warns that ties at the cutoff are order
// sensitive. Here the ranking key is (score descending, pool index ascending) and the chosen
// ids are written in ascending order, so the result is unique.
//
// One 1024-thread block per row. Thread t keeps the order-preserving 32-bit keys of pools
// [t*KPT, t*KPT + KPT) in registers (key 0 marks a non-candidate; every candidate maps above
// it). When there are more candidates than Kw, a most-significant-digit radix select (four
// 8-bit passes, LDS histogram) finds the Kw-th largest key K*. Every key above K* is taken,
// plus the lowest-index keys equal to K* (an exclusive prefix count of equal keys in pool
// order), and a block prefix sum of per-thread counts writes the ids in ascending order.
// Non-candidates never enter a histogram.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

constexpr int kThreads = 1024;

template <int KPT>
__global__ __launch_bounds__(kThreads) void topk_pools_kernel(int P, int Kw,
                                                              const float *__restrict__ scores,
                                                              const uint8_t *__restrict__ cand,
                                                              int32_t *__restrict__ sel) {
    __shared__ int scratch[kThreads / kWave + 1];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t pick[2];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const float *srow = scores + (size_t)r * P;
    const uint8_t *crow = cand + (size_t)r * P;
    const int base = tid * KPT;

    uint32_t key[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int p = base + i;
        key[i] = (p < P && crow[p]) ? ordered_key(srow[p]) : 0u;
    }
    int nc = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) nc += key[i] != 0u;
    const int n_cand = block_sum<kThreads>(nc, scratch);
    const int take = n_cand < Kw ? n_cand : Kw;

    uint32_t thr = 0u;  // take every key > thr, plus `need` of the keys == thr
    int need = 0;
    if (n_cand > Kw) {
        uint32_t prefix = 0u, pmask = 0u;
        int k = Kw;
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0u;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < KPT; ++i)
                if (key[i] != 0u && (key[i] & pmask) == prefix)
                    atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
            __syncthreads();
            if (tid < kWave) {
                // lane l covers digits 255-4l .. 252-4l, scanned from the top
                const int d0 = 255 - 4 * tid;
                const uint32_t c0 = hist[d0], c1 = hist[d0 - 1], c2 = hist[d0 - 2], c3 = hist[d0 - 3];
                const uint32_t s = c0 + c1 + c2 + c3;
                uint32_t inc = s;
#pragma unroll
                for (int d = 1; d < kWave; d <<= 1) {
                    const uint32_t o = __shfl_up(inc, d, kWave);
                    if (tid >= d) inc += o;
                }
                const uint32_t above = inc - s;
                const uint32_t kk = (uint32_t)k;
                if (above < kk && kk <= inc) {
                    uint32_t a = above;
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

    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        gt += key[i] > thr;
        eq += key[i] == thr && key[i] != 0u;
    }
    int eq_total;
    const int eq_before = block_exclusive_scan<kThreads>(eq, scratch, &eq_total);
    int take_eq = need - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
    int total;
    int o = block_exclusive_scan<kThreads>(gt + take_eq, scratch, &total);
    int32_t *orow = sel + (size_t)r * Kw;
    int eq_seen = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        bool s = key[i] > thr;
        if (key[i] == thr && key[i] != 0u) {
            s = eq_seen < take_eq;
            ++eq_seen;
        }
        if (s && o < Kw) orow[o++] = base + i;
    }
    for (int i = take + tid; i < Kw; i += kThreads) orow[i] = -1;
}

template <int KPT>
hipError_t launch_kpt(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                      int32_t *sel, hipStream_t stream) {
    hipLaunchKernelGGL(topk_pools_kernel<KPT>, dim3(Q), dim3(kThreads), 0, stream, P, Kw, scores,
                       cand, sel);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk_pools(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                             int32_t *sel, hipStream_t stream) {
    if (Q == 0 || Kw == 0) return hipSuccess;
    if (P <= kThreads * 1) return launch_kpt<1>(Q, P, Kw, scores, cand, sel, stream);
    if (P <= kThreads * 2) return launch_kpt<2>(Q, P, Kw, scores, cand, sel, stream);
    if (P <= kThreads * 4) return launch_kpt<4>(Q, P, Kw, scores, cand, sel, stream);
    if (P <= kThreads * 8) return launch_kpt<8>(Q, P, Kw, scores, cand, sel, stream);
    if (P <= kThreads * 16) return launch_kpt<16>(Q, P, Kw, scores, cand, sel, stream);
    if (P <= kThreads * 32) return launch_kpt<32>(Q, P, Kw, scores, cand, sel, stream);
    if (P <= kThreads * 64) return launch_kpt<64>(Q, P, Kw, scores, cand, sel, stream);
    return hipErrorInvalidValue;
}

}  // namespace dsa

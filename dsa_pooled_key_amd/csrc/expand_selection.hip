// expand_selection.hip -- selected pools -> token ids.
//
// mod.rs, "Shape of the pipeline" and "Checkpoint and kernel facts": [Q, out_width] token
// ids with -1 for invalid, every slot written. One thread per output slot computes that
// slot's final value (a token of a selected pool, a valid tail token, or -1) and stores it
// once, which writes the whole row without a separate -1 pass. Ids outside [0, P), rows whose
// sequence is out of range, and tail tokens outside [0, S) all give -1.
#include "dsa_device.hpp"
#include "dsa_launch.hpp"

namespace dsa {
namespace {

__global__ __launch_bounds__(256) void expand_selection_kernel(
    int Kw, int KP, int topk, int W, int tail, int B, int S, int first_key, int P,
    const int32_t *__restrict__ sel, const int32_t *__restrict__ row_seq,
    const int32_t *__restrict__ row_pos, const uint8_t *__restrict__ valid,
    int32_t *__restrict__ token_ids) {
    const int r = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= W) return;
    int v = -1;
    if (i < topk) {
        const int j = i / KP;
        if (j < Kw) {
            const int p = sel[(size_t)r * Kw + j];
            if (p >= 0 && p < P) v = first_key + p * KP + (i - j * KP);
        }
    } else if (tail) {
        const int b = row_seq[r];
        const long long pos = row_pos[r];
        if (b >= 0 && b < B && pos + 1 > first_key) {
            const long long start = first_key + ((pos + 1 - first_key) / KP) * KP;
            const long long t = start + (i - topk);
            if (t <= pos && t < S && valid[(size_t)b * S + t]) v = (int)t;
        }
    }
    token_ids[(size_t)r * W + i] = v;
}

}  // namespace

hipError_t launch_expand_selection(int Q, int Kw, int KP, int topk, int W, bool tail, int B,
                                   int S, int first_key, int P, const int32_t *sel,
                                   const int32_t *row_seq, const int32_t *row_pos,
                                   const uint8_t *valid, int32_t *token_ids, hipStream_t stream) {
    if (Q == 0 || W == 0) return hipSuccess;
    hipLaunchKernelGGL(expand_selection_kernel, dim3((W + 255) / 256, Q), dim3(256), 0, stream, Kw,
                       KP, topk, W, tail ? 1 : 0, B, S, first_key, P, sel, row_seq, row_pos, valid,
                       token_ids);
    return hipGetLastError();
}

}  // namespace dsa

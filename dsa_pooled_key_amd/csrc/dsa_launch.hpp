// dsa_launch.hpp -- internal launchers, one per kernel family. Arguments are already
// checked by the C ABI layer (dsa_api.cpp); each launcher returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// key_scales NULL: bf16 pooled keys; else fp8 e4m3 pooled keys with per-pool f32 scales.
hipError_t launch_kpool_compress(int B, int S, int D, int KP, int first_key, int P,
                                 const uint16_t *k, const uint16_t *gate, const float *ape,
                                 const uint8_t *valid, void *pool_keys, float *key_scales,
                                 uint8_t *pool_valid, hipStream_t stream);
// The pool each sequence's new token completes (key_scales NULL: bf16 keys, else fp8), and
// its id appended to the compacted list when valid.
hipError_t launch_pool_append(int B, int S, int D, int KP, int first_key, int P,
                              const int32_t *pos, const uint16_t *k, const uint16_t *gate,
                              const float *ape, const uint8_t *valid, void *pool_keys,
                              float *key_scales, uint8_t *pool_valid, int32_t *ids,
                              int32_t *n_valid, hipStream_t stream);
// LayerNorm with a bias over bf16 rows of D, in place (D/8 a power of two up to 64).
hipError_t launch_layer_norm(long long rows, int D, uint16_t *x, const uint16_t *weight,
                             const uint16_t *bias, float eps, hipStream_t stream);
// Staged rows to their positions, marked valid; decode geometry from the live lengths.
hipError_t launch_indexer_store(int B, int S, int D, const int32_t *pos, const uint16_t *k_row,
                                const uint16_t *gate_row, uint16_t *k_cache, uint16_t *gate_cache,
                                uint8_t *valid, hipStream_t stream);
hipError_t launch_write_geom(int B, const int32_t *seq_len, int32_t *row_seq, int32_t *row_pos,
                             hipStream_t stream);
// The dense masked cross-check: token mask of a selection; attention over every masked token.
hipError_t launch_topk_to_mask(int Q, int W, int S, const int32_t *token_ids, uint8_t *mask,
                               hipStream_t stream);
hipError_t launch_masked_attn(int Q, int H, int S, int B, float sm_scale, const uint16_t *q_abs,
                              const uint8_t *mask, const int32_t *row_seq, const void *kv,
                              bool kv_fp8, const float *kv_scales, int64_t kv_rows,
                              const int32_t *block_table, int max_blocks, int block_size,
                              float *out, float *lse, hipStream_t stream);
// Rows of n values (bf16 or f32) -> e4m3 codes and per-row f32 scales.
hipError_t launch_quantize_rows(long long rows, int n, const void *src, bool f32_src,
                                uint8_t *codes, float *scales, hipStream_t stream);

hipError_t launch_compact_pools(int B, int P, const uint8_t *pool_valid, int32_t *ids,
                                int32_t *n_valid, hipStream_t stream);

hipError_t launch_index_scores(int Q, int B, int P, int Hi, int D, int KP, int first_key,
                               float scale, const uint16_t *q, const float *w,
                               const int32_t *row_seq, const int32_t *row_pos, const void *keys,
                               bool key_fp8, const float *key_scales, const int32_t *ids,
                               const int32_t *n_valid, float *scores, uint8_t *cand,
                               hipStream_t stream);
hipError_t launch_index_scores_valid(int Q, int B, int P, int Hi, int D, int KP, int first_key,
                                     float scale, const uint16_t *q, const float *w,
                                     const int32_t *row_seq, const int32_t *row_pos,
                                     const void *keys, bool key_fp8, const float *key_scales,
                                     const uint8_t *pool_valid, float *scores, uint8_t *cand,
                                     hipStream_t stream);

// Largest row length the top-k kernel keeps in registers.
constexpr int kTopkMaxPools = 65536;
// Workspace of the two-stage selection for few long rows (0 when one block a row runs).
size_t topk_workspace_bytes(int Q, int P, int Kw);
hipError_t launch_topk_pools(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                             int32_t *sel, void *ws, size_t ws_bytes, hipStream_t stream);

// Top-k and token-id expansion in one kernel (same results as the two calls in sequence).
hipError_t launch_topk_expand(int Q, int P, int Kw, const float *scores, const uint8_t *cand,
                              int32_t *sel, int KP, int topk, int W, bool tail, int B, int S,
                              int first_key, const int32_t *row_seq, const int32_t *row_pos,
                              const uint8_t *valid, int32_t *token_ids, void *ws,
                              size_t ws_bytes, hipStream_t stream);

hipError_t launch_expand_selection(int Q, int Kw, int KP, int topk, int W, bool tail, int B,
                                   int S, int first_key, int P, const int32_t *sel,
                                   const int32_t *row_seq, const int32_t *row_pos,
                                   const uint8_t *valid, int32_t *token_ids, hipStream_t stream);

// Sparse MLA split limits: token slots one block resolves up front, splits per row.
constexpr int kMlaMaxSplit = 2048;
constexpr int kMlaMaxSplits = 16;
static_assert(kMlaMaxSplit * kMlaMaxSplits >= DSA_MAX_MLA_WIDTH, "widest selection must fit");

struct MlaPlan {
    int groups;      // 32-head groups
    int splits;      // token splits per (row, group)
    int split_len;   // token slots per split (multiple of 32)
    int teams;       // splits per block (1 or 2)
    int parts;       // blocks per (row, group): ceil(splits / teams)
    size_t ws_bytes; // partial results for parts > 1
};
MlaPlan plan_sparse_mla(int Q, int W, int H);
// Compute units of the current device (queried once per device).
hipError_t device_cu_count(int *cus);
// Size of the fixed device scratch behind dsa_sparse_mla_decode_noalloc, and its address on
// the current device (looked up once per device, then cached).
constexpr size_t kMlaNoallocScratchBytes = DSA_MLA_NOALLOC_SCRATCH_BYTES;
hipError_t mla_noalloc_scratch(void **ptr);
hipError_t launch_sparse_mla(const MlaPlan &plan, int Q, int W, int H, int B, float sm_scale,
                             const uint16_t *q_abs, const int32_t *token_ids,
                             const int32_t *row_seq, const void *kv, bool kv_fp8,
                             const float *kv_scales, int64_t kv_rows, int S,
                             const int32_t *block_table, int max_blocks, int block_size,
                             float *out, float *lse, void *ws, hipStream_t stream);

// Measurement only (stream_read.hip): every 16-byte word of buf read once; sink gets the XOR.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int blocks,
                              hipStream_t stream);
hipError_t launch_empty(int blocks, hipStream_t stream);
hipError_t launch_mfma_rate(int kind, int blocks, int iters, float *out, hipStream_t stream);

}  // namespace dsa

// dsa_api.cpp -- the extern "C" entry points of libdsa declared in include/dsa.h.
//
// Every call checks its arguments on the host first (null pointers, sizes, alignment,
// the config rules of mod.rs Glm5NextDsaConfig::validate) and launches nothing on a refusal.
// Kernels are enqueued on the caller's stream; nothing here allocates or synchronizes.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dsa.h"
#include "dsa_host.hpp"
#include "dsa_launch.hpp"

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace dsa_host {
int set_error(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}
void clear_error() { g_err[0] = 0; }
}  // namespace dsa_host

namespace {

using dsa_host::clear_error;
using dsa_host::set_error;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return DSA_OK;
    return set_error(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The six refusals of mod.rs Glm5NextDsaConfig::validate, in the page's order.
int check_config(const dsa_config *c) {
    if (!c) return set_error(DSA_ERR_NULL_ARG, "config is NULL");
    if (c->index_kpool == 0 || c->index_topk == 0)
        return set_error(DSA_ERR_KPOOL_OR_TOPK_ZERO,
                    "index_kpool and index_topk must both be positive (got %d and %d)",
                    c->index_kpool, c->index_topk);
    if (c->index_kpool < 0 || c->index_topk < 0)
        return set_error(DSA_ERR_BAD_SIZE, "index_kpool and index_topk must be positive");
    if (c->index_topk % c->index_kpool != 0)
        return set_error(DSA_ERR_TOPK_NOT_MULTIPLE,
                    "index_topk %d is not a whole number of pools of %d tokens", c->index_topk,
                    c->index_kpool);
    if (c->index_kpool > DSA_MAX_KPOOL)
        return set_error(DSA_ERR_KPOOL_GT_MAX,
                    "index_kpool %d is above the %d pool slots the pooling kernel holds",
                    c->index_kpool, DSA_MAX_KPOOL);
    if (c->kv_lora_rank == 0) return set_error(DSA_ERR_KV_LORA_ZERO, "kv_lora_rank is 0; MLA needs a latent");
    if (c->kv_lora_rank != DSA_LATENT_DIM)
        return set_error(DSA_ERR_KV_LORA_NOT_512,
                    "kv_lora_rank %d differs from the %d-wide latent the decode kernels read",
                    c->kv_lora_rank, DSA_LATENT_DIM);
    if (c->heads == 0) return set_error(DSA_ERR_ZERO_HEADS, "no attention heads on this device");
    if (c->heads < 0) return set_error(DSA_ERR_BAD_SIZE, "heads is negative");
    return DSA_OK;
}

int check_index_geometry(const dsa_config *c) {
    if (c->index_heads <= 0 || c->index_heads > DSA_MAX_INDEX_HEADS)
        return set_error(DSA_ERR_UNSUPPORTED, "index_heads %d outside 1..%d", c->index_heads,
                    DSA_MAX_INDEX_HEADS);
    if (c->index_head_dim != 32 && c->index_head_dim != 64 && c->index_head_dim != 128)
        return set_error(DSA_ERR_UNSUPPORTED, "index_head_dim %d is not 32, 64 or 128",
                    c->index_head_dim);
    return DSA_OK;
}

int64_t num_pools(int64_t S, int64_t first_key, int64_t kpool) {
    if (S <= first_key) return 0;
    return (S - first_key) / kpool;
}

int64_t select_k(const dsa_config *c, int64_t n_pools) {
    const int64_t k = c->index_topk / c->index_kpool;
    return k < n_pools ? k : n_pools;
}

int64_t out_width(const dsa_config *c) {
    return (int64_t)c->index_topk + (c->always_select_tail ? c->index_kpool - 1 : 0);
}

}  // namespace

extern "C" {

const char *dsa_last_error(void) { return g_err; }

const char *dsa_version(void) { return "dsa 0.1.0 gfx950"; }

int dsa_config_validate(const dsa_config *cfg) {
    clear_error();
    return check_config(cfg);
}

int64_t dsa_select_k(const dsa_config *cfg, int64_t n_pools) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    if (n_pools < 0) return set_error(DSA_ERR_BAD_SIZE, "n_pools is negative");
    return select_k(cfg, n_pools);
}

int64_t dsa_out_width(const dsa_config *cfg) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    return out_width(cfg);
}

int64_t dsa_num_pools(int64_t S, int64_t first_key, int64_t kpool) {
    clear_error();
    if (kpool <= 0 || S < 0 || first_key < 0)
        return set_error(DSA_ERR_BAD_SIZE, "num_pools needs kpool > 0 and non-negative S, first_key");
    return num_pools(S, first_key, kpool);
}

int dsa_kpool_compress(const dsa_config *cfg, int B, int S, int first_key, const void *k,
                       const void *gate, const float *ape, const uint8_t *valid, void *pool_keys,
                       uint8_t *pool_valid, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    const int D = cfg->index_head_dim;
    if (D <= 0 || D % 8 != 0 || D > 1024)
        return set_error(DSA_ERR_UNSUPPORTED, "index_head_dim %d must be a positive multiple of 8", D);
    if (B < 0 || S < 0 || first_key < 0) return set_error(DSA_ERR_BAD_SIZE, "negative B, S or first_key");
    const int64_t P = num_pools(S, first_key, cfg->index_kpool);
    if ((int64_t)B * P == 0) return DSA_OK;
    if (!k || !gate || !ape || !valid || !pool_keys || !pool_valid)
        return set_error(DSA_ERR_NULL_ARG, "kpool_compress: a buffer is NULL");
    if (!aligned(k, 16) || !aligned(gate, 16) || !aligned(pool_keys, 16) || !aligned(ape, 16))
        return set_error(DSA_ERR_BAD_SIZE, "kpool_compress: k, gate, pool_keys and ape need 16-byte alignment");
    return hip_status(dsa::launch_kpool_compress(B, S, D, cfg->index_kpool, first_key, (int)P,
                                                 static_cast<const uint16_t *>(k),
                                                 static_cast<const uint16_t *>(gate), ape, valid,
                                                 pool_keys, nullptr, pool_valid, stream),
                      "kpool_compress launch");
}

int dsa_kpool_compress_fp8(const dsa_config *cfg, int B, int S, int first_key, const void *k,
                           const void *gate, const float *ape, const uint8_t *valid,
                           uint8_t *pool_keys, float *pool_key_scales, uint8_t *pool_valid,
                           hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    const int D = cfg->index_head_dim;
    if (D < 8 || D > 512 || (D & (D - 1)) != 0)
        return set_error(DSA_ERR_UNSUPPORTED, "kpool_compress_fp8: index_head_dim %d must be a power of two in [8, 512]", D);
    if (B < 0 || S < 0 || first_key < 0) return set_error(DSA_ERR_BAD_SIZE, "negative B, S or first_key");
    const int64_t P = num_pools(S, first_key, cfg->index_kpool);
    if ((int64_t)B * P == 0) return DSA_OK;
    if (!k || !gate || !ape || !valid || !pool_keys || !pool_key_scales || !pool_valid)
        return set_error(DSA_ERR_NULL_ARG, "kpool_compress_fp8: a buffer is NULL");
    if (!aligned(k, 16) || !aligned(gate, 16) || !aligned(pool_keys, 8) || !aligned(ape, 16))
        return set_error(DSA_ERR_BAD_SIZE, "kpool_compress_fp8: k, gate and ape need 16-byte alignment, pool_keys 8-byte");
    return hip_status(dsa::launch_kpool_compress(B, S, D, cfg->index_kpool, first_key, (int)P,
                                                 static_cast<const uint16_t *>(k),
                                                 static_cast<const uint16_t *>(gate), ape, valid,
                                                 pool_keys, pool_key_scales, pool_valid, stream),
                      "kpool_compress_fp8 launch");
}

int dsa_topk_to_mask(int Q, int W, int S, const int32_t *token_ids, uint8_t *mask,
                     hipStream_t stream) {
    clear_error();
    if (Q < 0 || W < 0 || S < 0) return set_error(DSA_ERR_BAD_SIZE, "topk_to_mask: negative size");
    if (Q == 0 || S == 0) return DSA_OK;
    if (!mask || (W > 0 && !token_ids)) return set_error(DSA_ERR_NULL_ARG, "topk_to_mask: a buffer is NULL");
    return hip_status(dsa::launch_topk_to_mask(Q, W, S, token_ids, mask, stream), "topk_to_mask launch");
}

int dsa_mla_masked_attn(const dsa_config *cfg, int Q, int S, int B, float sm_scale,
                        const void *q_abs, const uint8_t *mask, const int32_t *row_seq,
                        const void *kv, dsa_dtype kv_dtype, const float *kv_scales,
                        int64_t kv_rows, const int32_t *block_table, int max_blocks,
                        int block_size, float *out, float *lse, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    if (Q < 0 || S < 0 || B < 0 || kv_rows < 0) return set_error(DSA_ERR_BAD_SIZE, "negative size");
    if (S > DSA_MASKED_ATTN_MAX_KEYS)
        return set_error(DSA_ERR_UNSUPPORTED, "mla_masked_attn: S = %d above the %d keys of the score row",
                    S, DSA_MASKED_ATTN_MAX_KEYS);
    if (kv_dtype != DSA_BF16 && kv_dtype != DSA_FP8_E4M3)
        return set_error(DSA_ERR_BAD_DTYPE, "mla_masked_attn: latent must be bf16 or fp8 e4m3");
    if (kv_rows > INT32_MAX) return set_error(DSA_ERR_UNSUPPORTED, "mla_masked_attn: kv_rows above 2^31 - 1");
    if (Q == 0 || cfg->heads == 0) return DSA_OK;
    const bool fp8 = kv_dtype == DSA_FP8_E4M3;
    if (!q_abs || !row_seq || !out || (S > 0 && !mask))
        return set_error(DSA_ERR_NULL_ARG, "mla_masked_attn: a buffer is NULL");
    if (kv_rows > 0 && !kv) return set_error(DSA_ERR_NULL_ARG, "mla_masked_attn: kv is NULL");
    if (fp8 && kv_rows > 0 && !kv_scales)
        return set_error(DSA_ERR_NULL_ARG, "mla_masked_attn: fp8 latent needs kv_scales");
    if (block_table && (block_size <= 0 || max_blocks < 0))
        return set_error(DSA_ERR_BAD_SIZE, "mla_masked_attn: paged latent needs block_size > 0");
    if (!aligned(q_abs, 16) || (kv && !aligned(kv, 16)) || !aligned(out, 8))
        return set_error(DSA_ERR_BAD_SIZE, "mla_masked_attn: q_abs and kv need 16-byte alignment");
    return hip_status(dsa::launch_masked_attn(Q, cfg->heads, S, B, sm_scale,
                                              static_cast<const uint16_t *>(q_abs), mask, row_seq, kv,
                                              fp8, kv_scales, kv_rows, block_table, max_blocks,
                                              block_size, out, lse, stream),
                      "mla_masked_attn launch");
}

int dsa_k_norm(int64_t rows, int D, void *x, const void *weight, const void *bias, float eps,
               hipStream_t stream) {
    clear_error();
    if (rows < 0 || D <= 0) return set_error(DSA_ERR_BAD_SIZE, "k_norm: rows >= 0 and D > 0 needed");
    if (D % 8 != 0 || D > 512 || ((D / 8) & (D / 8 - 1)) != 0)
        return set_error(DSA_ERR_UNSUPPORTED, "k_norm: D = %d must be 8 times a power of two, at most 512", D);
    if (!(eps >= 0.0f)) return set_error(DSA_ERR_BAD_SIZE, "k_norm: eps must be >= 0");
    if (rows > INT32_MAX) return set_error(DSA_ERR_UNSUPPORTED, "k_norm: rows above 2^31 - 1");
    if (rows == 0) return DSA_OK;
    if (!x || !weight || !bias) return set_error(DSA_ERR_NULL_ARG, "k_norm: a buffer is NULL");
    if (!aligned(x, 16) || !aligned(weight, 16) || !aligned(bias, 16))
        return set_error(DSA_ERR_BAD_SIZE, "k_norm: x, weight and bias need 16-byte alignment");
    return hip_status(dsa::launch_layer_norm((long long)rows, D, static_cast<uint16_t *>(x),
                                             static_cast<const uint16_t *>(weight),
                                             static_cast<const uint16_t *>(bias), eps, stream),
                      "k_norm launch");
}

int dsa_indexer_store(int B, int S, int D, const int32_t *pos, const void *k_row, const void *gate_row,
                      void *k_cache, void *gate_cache, uint8_t *valid, hipStream_t stream) {
    clear_error();
    if (B < 0 || S < 0 || D <= 0) return set_error(DSA_ERR_BAD_SIZE, "indexer_store: B, S >= 0 and D > 0 needed");
    if (D % 8 != 0) return set_error(DSA_ERR_UNSUPPORTED, "indexer_store: D = %d must be a multiple of 8", D);
    if (B == 0 || S == 0) return DSA_OK;
    if (!pos || !k_row || !gate_row || !k_cache || !gate_cache || !valid)
        return set_error(DSA_ERR_NULL_ARG, "indexer_store: a buffer is NULL");
    if (!aligned(k_row, 16) || !aligned(gate_row, 16) || !aligned(k_cache, 16) || !aligned(gate_cache, 16))
        return set_error(DSA_ERR_BAD_SIZE, "indexer_store: rows and caches need 16-byte alignment");
    return hip_status(dsa::launch_indexer_store(B, S, D, pos, static_cast<const uint16_t *>(k_row),
                                                static_cast<const uint16_t *>(gate_row),
                                                static_cast<uint16_t *>(k_cache),
                                                static_cast<uint16_t *>(gate_cache), valid, stream),
                      "indexer_store launch");
}

int dsa_write_geom(int B, const int32_t *seq_len, int32_t *row_seq, int32_t *row_pos, hipStream_t stream) {
    clear_error();
    if (B < 0) return set_error(DSA_ERR_BAD_SIZE, "write_geom: negative B");
    if (B == 0) return DSA_OK;
    if (!seq_len || !row_seq || !row_pos) return set_error(DSA_ERR_NULL_ARG, "write_geom: a buffer is NULL");
    return hip_status(dsa::launch_write_geom(B, seq_len, row_seq, row_pos, stream), "write_geom launch");
}

int dsa_pool_append(const dsa_config *cfg, int B, int S, int first_key, const int32_t *pos,
                    const void *k, const void *gate, const float *ape, const uint8_t *valid,
                    void *pool_keys, float *pool_key_scales, uint8_t *pool_valid, int32_t *ids,
                    int32_t *n_valid, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    const int D = cfg->index_head_dim;
    if (D < 8 || D > 512 || (D & (D - 1)) != 0)
        return set_error(DSA_ERR_UNSUPPORTED, "pool_append: index_head_dim %d must be a power of two in [8, 512]", D);
    if (B < 0 || S < 0 || first_key < 0) return set_error(DSA_ERR_BAD_SIZE, "negative B, S or first_key");
    const int64_t P = num_pools(S, first_key, cfg->index_kpool);
    if ((int64_t)B * P == 0) return DSA_OK;
    if (!pos || !k || !gate || !ape || !valid || !pool_keys || !pool_valid || !ids || !n_valid)
        return set_error(DSA_ERR_NULL_ARG, "pool_append: a buffer is NULL");
    if (!aligned(k, 16) || !aligned(gate, 16) || !aligned(ape, 16) ||
        !aligned(pool_keys, pool_key_scales ? 8 : 16))
        return set_error(DSA_ERR_BAD_SIZE, "pool_append: k, gate, ape and pool_keys need 16-byte alignment (8 for fp8 keys)");
    return hip_status(dsa::launch_pool_append(B, S, D, cfg->index_kpool, first_key, (int)P, pos,
                                              static_cast<const uint16_t *>(k),
                                              static_cast<const uint16_t *>(gate), ape, valid, pool_keys,
                                              pool_key_scales, pool_valid, ids, n_valid, stream),
                      "pool_append launch");
}

int dsa_quantize_rows_fp8(int64_t rows, int n, const void *src, dsa_dtype src_dtype, uint8_t *codes,
                          float *scales, hipStream_t stream) {
    clear_error();
    if (rows < 0 || n <= 0) return set_error(DSA_ERR_BAD_SIZE, "quantize_rows_fp8: rows >= 0 and n > 0 needed");
    if (n % 8 != 0 || n > 4096)
        return set_error(DSA_ERR_UNSUPPORTED, "quantize_rows_fp8: n = %d must be a multiple of 8 up to 4096", n);
    if (src_dtype != DSA_BF16 && src_dtype != DSA_F32)
        return set_error(DSA_ERR_BAD_DTYPE, "quantize_rows_fp8: source must be bf16 or f32");
    if (rows > INT32_MAX) return set_error(DSA_ERR_UNSUPPORTED, "quantize_rows_fp8: rows above 2^31 - 1");
    if (rows == 0) return DSA_OK;
    if (!src || !codes || !scales) return set_error(DSA_ERR_NULL_ARG, "quantize_rows_fp8: a buffer is NULL");
    if (!aligned(src, 16) || !aligned(codes, 8))
        return set_error(DSA_ERR_BAD_SIZE, "quantize_rows_fp8: src needs 16-byte and codes 8-byte alignment");
    return hip_status(dsa::launch_quantize_rows((long long)rows, n, src, src_dtype == DSA_F32, codes,
                                                scales, stream),
                      "quantize_rows_fp8 launch");
}

int dsa_compact_pools(int B, int P, const uint8_t *pool_valid, int32_t *ids, int32_t *n_valid,
                      hipStream_t stream) {
    clear_error();
    if (B < 0 || P < 0) return set_error(DSA_ERR_BAD_SIZE, "negative B or P");
    if (B == 0) return DSA_OK;
    if (!n_valid || (P > 0 && (!pool_valid || !ids)))
        return set_error(DSA_ERR_NULL_ARG, "compact_pools: a buffer is NULL");
    return hip_status(dsa::launch_compact_pools(B, P, pool_valid, ids, n_valid, stream),
                      "compact_pools launch");
}

int dsa_index_scores(const dsa_config *cfg, int Q, int B, int P, int first_key, float scale,
                     const void *q, const float *w, const int32_t *row_seq,
                     const int32_t *row_pos, const void *keys, dsa_dtype key_dtype,
                     const float *key_scales, const int32_t *ids, const int32_t *n_valid,
                     float *scores, uint8_t *cand, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_index_geometry(cfg))) return rc;
    if (Q < 0 || B < 0 || P < 0 || first_key < 0) return set_error(DSA_ERR_BAD_SIZE, "negative size");
    if (key_dtype != DSA_BF16 && key_dtype != DSA_FP8_E4M3)
        return set_error(DSA_ERR_BAD_DTYPE, "index_scores: keys must be bf16 or fp8 e4m3");
    if (Q == 0 || P == 0) return DSA_OK;
    if (B == 0) return set_error(DSA_ERR_BAD_SIZE, "index_scores: rows need at least one sequence");
    if (!q || !w || !row_seq || !row_pos || !keys || !ids || !n_valid || !scores || !cand)
        return set_error(DSA_ERR_NULL_ARG, "index_scores: a buffer is NULL");
    const bool fp8 = key_dtype == DSA_FP8_E4M3;
    if (fp8 && !key_scales) return set_error(DSA_ERR_NULL_ARG, "index_scores: fp8 keys need key_scales");
    if (!aligned(q, 16) || !aligned(keys, 16))
        return set_error(DSA_ERR_BAD_SIZE, "index_scores: q and keys need 16-byte alignment");
    if ((long long)first_key + (long long)P * cfg->index_kpool > 0x7fffffffLL)
        return set_error(DSA_ERR_BAD_SIZE, "index_scores: token positions exceed int32");
    return hip_status(dsa::launch_index_scores(Q, B, P, cfg->index_heads, cfg->index_head_dim,
                                               cfg->index_kpool, first_key, scale,
                                               static_cast<const uint16_t *>(q), w, row_seq,
                                               row_pos, keys, fp8, key_scales, ids, n_valid,
                                               scores, cand, stream),
                      "index_scores launch");
}

int dsa_compact_index_scores(const dsa_config *cfg, int Q, int B, int P, int first_key,
                             float scale, const void *q, const float *w, const int32_t *row_seq,
                             const int32_t *row_pos, const void *keys, dsa_dtype key_dtype,
                             const float *key_scales, const uint8_t *pool_valid, float *scores,
                             uint8_t *cand, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_index_geometry(cfg))) return rc;
    if (Q < 0 || B < 0 || P < 0 || first_key < 0) return set_error(DSA_ERR_BAD_SIZE, "negative size");
    if (key_dtype != DSA_BF16 && key_dtype != DSA_FP8_E4M3)
        return set_error(DSA_ERR_BAD_DTYPE, "compact_index_scores: keys must be bf16 or fp8 e4m3");
    if (Q == 0 || P == 0) return DSA_OK;
    if (B == 0) return set_error(DSA_ERR_BAD_SIZE, "compact_index_scores: rows need at least one sequence");
    if (!q || !w || !row_seq || !row_pos || !keys || !pool_valid || !scores || !cand)
        return set_error(DSA_ERR_NULL_ARG, "compact_index_scores: a buffer is NULL");
    const bool fp8 = key_dtype == DSA_FP8_E4M3;
    if (fp8 && !key_scales)
        return set_error(DSA_ERR_NULL_ARG, "compact_index_scores: fp8 keys need key_scales");
    if (!aligned(q, 16) || !aligned(keys, 16))
        return set_error(DSA_ERR_BAD_SIZE, "compact_index_scores: q and keys need 16-byte alignment");
    if ((long long)first_key + (long long)P * cfg->index_kpool > 0x7fffffffLL)
        return set_error(DSA_ERR_BAD_SIZE, "compact_index_scores: token positions exceed int32");
    return hip_status(dsa::launch_index_scores_valid(Q, B, P, cfg->index_heads, cfg->index_head_dim,
                                                     cfg->index_kpool, first_key, scale,
                                                     static_cast<const uint16_t *>(q), w, row_seq,
                                                     row_pos, keys, fp8, key_scales, pool_valid,
                                                     scores, cand, stream),
                      "compact_index_scores launch");
}

size_t dsa_topk_workspace(const dsa_config *cfg, int Q, int P) {
    clear_error();
    if (check_config(cfg) || Q < 0 || P < 0 || P > dsa::kTopkMaxPools) return 0;
    return dsa::topk_workspace_bytes(Q, P, (int)select_k(cfg, P));
}

size_t dsa_topk_pools_workspace(const dsa_config *cfg, int Q, int P) {
    return dsa_topk_workspace(cfg, Q, P);
}

int dsa_topk_pools(const dsa_config *cfg, int Q, int P, const float *scores, const uint8_t *cand,
                   int32_t *sel, void *ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    if (Q < 0 || P < 0) return set_error(DSA_ERR_BAD_SIZE, "negative Q or P");
    if (P > dsa::kTopkMaxPools)
        return set_error(DSA_ERR_UNSUPPORTED, "topk_pools: rows of %d pools exceed the %d this kernel keeps",
                    P, dsa::kTopkMaxPools);
    const int Kw = (int)select_k(cfg, P);
    if (Q == 0 || Kw == 0) return DSA_OK;
    if (!scores || !cand || !sel) return set_error(DSA_ERR_NULL_ARG, "topk_pools: a buffer is NULL");
    if (ws_bytes > 0 && (!ws || !aligned(ws, 16)))
        return set_error(DSA_ERR_WORKSPACE, "topk_pools: a workspace needs a 16-byte aligned pointer");
    return hip_status(dsa::launch_topk_pools(Q, P, Kw, scores, cand, sel, ws, ws_bytes, stream),
                      "topk_pools launch");
}

int dsa_expand_selection(const dsa_config *cfg, int Q, int Kw, int B, int S, int first_key,
                         const int32_t *sel, const int32_t *row_seq, const int32_t *row_pos,
                         const uint8_t *valid, int32_t *token_ids, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    if (Q < 0 || Kw < 0 || B < 0 || S < 0 || first_key < 0) return set_error(DSA_ERR_BAD_SIZE, "negative size");
    if ((int64_t)Kw * cfg->index_kpool > cfg->index_topk)
        return set_error(DSA_ERR_BAD_SIZE, "expand_selection: %d pools of %d tokens exceed index_topk %d", Kw,
                    cfg->index_kpool, cfg->index_topk);
    const int64_t W = out_width(cfg);
    if (Q == 0) return DSA_OK;
    const bool tail = cfg->always_select_tail != 0;
    if (!token_ids || (Kw > 0 && !sel) || (tail && (!row_seq || !row_pos || !valid)))
        return set_error(DSA_ERR_NULL_ARG, "expand_selection: a buffer is NULL");
    const int64_t P = num_pools(S, first_key, cfg->index_kpool);
    return hip_status(dsa::launch_expand_selection(Q, Kw, cfg->index_kpool, cfg->index_topk, (int)W,
                                                   tail, B, S, first_key, (int)P, sel, row_seq,
                                                   row_pos, valid, token_ids, stream),
                      "expand_selection launch");
}

int dsa_topk_expand(const dsa_config *cfg, int Q, int P, const float *scores, const uint8_t *cand,
                    int B, int S, int first_key, const int32_t *row_seq, const int32_t *row_pos,
                    const uint8_t *valid, int32_t *sel, int32_t *token_ids, void *ws,
                    size_t ws_bytes, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    if (Q < 0 || P < 0 || B < 0 || S < 0 || first_key < 0) return set_error(DSA_ERR_BAD_SIZE, "negative size");
    if (P > dsa::kTopkMaxPools)
        return set_error(DSA_ERR_UNSUPPORTED, "topk_expand: rows of %d pools exceed the %d this kernel keeps",
                    P, dsa::kTopkMaxPools);
    if (P > num_pools(S, first_key, cfg->index_kpool))
        return set_error(DSA_ERR_BAD_SIZE, "topk_expand: %d pools exceed the %lld that S = %d holds", P,
                    (long long)num_pools(S, first_key, cfg->index_kpool), S);
    const int Kw = (int)select_k(cfg, P);
    const int64_t W = out_width(cfg);
    if (Q == 0) return DSA_OK;
    const bool tail = cfg->always_select_tail != 0;
    if (!token_ids || (Kw > 0 && (!scores || !cand || !sel)) || (tail && (!row_seq || !row_pos || !valid)))
        return set_error(DSA_ERR_NULL_ARG, "topk_expand: a buffer is NULL");
    if (ws_bytes > 0 && (!ws || !aligned(ws, 16)))
        return set_error(DSA_ERR_WORKSPACE, "topk_expand: a workspace needs a 16-byte aligned pointer");
    return hip_status(dsa::launch_topk_expand(Q, P, Kw, scores, cand, sel, cfg->index_kpool,
                                              cfg->index_topk, (int)W, tail, B, S, first_key, row_seq,
                                              row_pos, valid, token_ids, ws, ws_bytes, stream),
                      "topk_expand launch");
}

size_t dsa_sparse_mla_decode_workspace(const dsa_config *cfg, int Q, int W) {
    clear_error();
    if (check_config(cfg) || Q < 0 || W < 0 || W > DSA_MAX_MLA_WIDTH) return 0;
    return dsa::plan_sparse_mla(Q, W, cfg->heads).ws_bytes;
}

}  // extern "C"

namespace {

// dsa_sparse_mla_decode and its no-allocation variant: the same checks and launches; with
// noalloc the split partials go to the library's fixed device scratch instead of ws.
int sparse_mla_decode_impl(const dsa_config *cfg, int Q, int W, int B, float sm_scale,
                           const void *q_abs, const int32_t *token_ids, const int32_t *row_seq,
                           const void *kv, dsa_dtype kv_dtype, const float *kv_scales,
                           int64_t kv_rows, int S, const int32_t *block_table, int max_blocks,
                           int block_size, float *out, float *lse, void *ws, size_t ws_bytes,
                           bool noalloc, hipStream_t stream) {
    clear_error();
    int rc = check_config(cfg);
    if (rc) return rc;
    if (Q < 0 || W < 0 || B < 0 || S < 0 || kv_rows < 0) return set_error(DSA_ERR_BAD_SIZE, "negative size");
    if (kv_dtype != DSA_BF16 && kv_dtype != DSA_FP8_E4M3)
        return set_error(DSA_ERR_BAD_DTYPE, "sparse_mla_decode: latent must be bf16 or fp8 e4m3");
    if (kv_rows > INT32_MAX)
        return set_error(DSA_ERR_UNSUPPORTED, "sparse_mla_decode: kv_rows above 2^31 - 1");
    if (W > DSA_MAX_MLA_WIDTH)
        return set_error(DSA_ERR_UNSUPPORTED, "sparse_mla_decode: W = %d above %d", W, DSA_MAX_MLA_WIDTH);
    if (Q == 0) return DSA_OK;
    const bool fp8 = kv_dtype == DSA_FP8_E4M3;
    if (!q_abs || !row_seq || !out || (W > 0 && !token_ids))
        return set_error(DSA_ERR_NULL_ARG, "sparse_mla_decode: a buffer is NULL");
    if (kv_rows > 0 && !kv) return set_error(DSA_ERR_NULL_ARG, "sparse_mla_decode: kv is NULL");
    if (fp8 && kv_rows > 0 && !kv_scales)
        return set_error(DSA_ERR_NULL_ARG, "sparse_mla_decode: fp8 latent needs kv_scales");
    if (block_table) {
        if (block_size <= 0 || max_blocks < 0)
            return set_error(DSA_ERR_BAD_SIZE, "sparse_mla_decode: paged latent needs block_size > 0");
    } else if (S <= 0 && W > 0) {
        // Contiguous rows are b*S + t: without a positive stride every sequence would read
        // sequence 0's rows.
        return set_error(DSA_ERR_BAD_SIZE, "sparse_mla_decode: a contiguous latent needs S > 0");
    }
    if (!aligned(q_abs, 16) || (kv && !aligned(kv, 16)) || !aligned(out, 16))
        return set_error(DSA_ERR_BAD_SIZE, "sparse_mla_decode: q_abs, kv and out need 16-byte alignment");
    const dsa::MlaPlan plan = dsa::plan_sparse_mla(Q, W, cfg->heads);
    if (noalloc) {
        if (plan.ws_bytes > dsa::kMlaNoallocScratchBytes)
            return set_error(DSA_ERR_WORKSPACE,
                             "sparse_mla_decode_noalloc: Q = %d, W = %d needs %zu bytes of split "
                             "partials, above the %zu-byte fixed scratch (use dsa_sparse_mla_decode "
                             "with a workspace)",
                             Q, W, plan.ws_bytes, dsa::kMlaNoallocScratchBytes);
        ws = nullptr;
        if (plan.ws_bytes > 0) {
            const hipError_t e = dsa::mla_noalloc_scratch(&ws);
            if (e != hipSuccess) return hip_status(e, "sparse_mla_decode_noalloc scratch lookup");
        }
    } else if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned(ws, 16))) {
        return set_error(DSA_ERR_WORKSPACE, "sparse_mla_decode: needs a 16-byte aligned workspace of %zu bytes",
                    plan.ws_bytes);
    }
    return hip_status(dsa::launch_sparse_mla(plan, Q, W, cfg->heads, B, sm_scale,
                                             static_cast<const uint16_t *>(q_abs), token_ids,
                                             row_seq, kv, fp8, kv_scales, kv_rows, S, block_table,
                                             max_blocks, block_size, out, lse, ws, stream),
                      "sparse_mla_decode launch");
}

}  // namespace

extern "C" {

int dsa_sparse_mla_decode(const dsa_config *cfg, int Q, int W, int B, float sm_scale,
                          const void *q_abs, const int32_t *token_ids, const int32_t *row_seq,
                          const void *kv, dsa_dtype kv_dtype, const float *kv_scales,
                          int64_t kv_rows, int S, const int32_t *block_table, int max_blocks,
                          int block_size, float *out, float *lse, void *ws, size_t ws_bytes,
                          hipStream_t stream) {
    return sparse_mla_decode_impl(cfg, Q, W, B, sm_scale, q_abs, token_ids, row_seq, kv, kv_dtype,
                                  kv_scales, kv_rows, S, block_table, max_blocks, block_size, out,
                                  lse, ws, ws_bytes, false, stream);
}

int dsa_sparse_mla_decode_noalloc(const dsa_config *cfg, int Q, int W, int B, float sm_scale,
                                  const void *q_abs, const int32_t *token_ids,
                                  const int32_t *row_seq, const void *kv, dsa_dtype kv_dtype,
                                  const float *kv_scales, int64_t kv_rows, int S,
                                  const int32_t *block_table, int max_blocks, int block_size,
                                  float *out, float *lse, hipStream_t stream) {
    return sparse_mla_decode_impl(cfg, Q, W, B, sm_scale, q_abs, token_ids, row_seq, kv, kv_dtype,
                                  kv_scales, kv_rows, S, block_table, max_blocks, block_size, out,
                                  lse, nullptr, 0, true, stream);
}

int dsa_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    clear_error();
    if (bytes == 0) return DSA_OK;
    if (!buf || !sink) return set_error(DSA_ERR_NULL_ARG, "stream_read: a buffer is NULL");
    if (bytes % 16 != 0 || !aligned(buf, 16) || !aligned(sink, 4))
        return set_error(DSA_ERR_BAD_SIZE, "stream_read: needs a 16-byte aligned buffer of a multiple of 16 bytes");
    return hip_status(dsa::launch_stream_read(buf, bytes, sink, 2048, stream), "stream_read launch");
}

int dsa_empty_launch(int blocks, hipStream_t stream) {
    clear_error();
    if (blocks < 1 || blocks > 65535)
        return set_error(DSA_ERR_BAD_SIZE, "empty_launch: blocks must be in 1..65535 (got %d)", blocks);
    return hip_status(dsa::launch_empty(blocks, stream), "empty launch");
}

int dsa_mfma_rate(int kind, int blocks, int iters, float *out, hipStream_t stream) {
    clear_error();
    if (kind < 0 || kind > 2 || blocks < 1 || blocks > 65535 || iters < 2 || iters % 2 != 0)
        return set_error(DSA_ERR_BAD_SIZE, "mfma_rate: kind 0..2, blocks 1..65535, iters even and >= 2");
    if (!out) return set_error(DSA_ERR_NULL_ARG, "mfma_rate: out is NULL");
    return hip_status(dsa::launch_mfma_rate(kind, blocks, iters, out, stream), "mfma_rate launch");
}

}  // extern "C"

/*
 * dsa.h -- C ABI of libdsa: the pooled-key DeepSeek Sparse Attention (DSA) indexer and the
 * absorbed-query NoPE MLA decode restricted to the selected tokens, for AMD Instinct MI355X
 * (gfx950).
 *
 * The pipeline follows the documentation pages of metrale_model_arch::glm5next_dsa, mod.rs,
 * module doc "Shape of the pipeline":
 *
 *   k, gate, valid, ape -> dsa_kpool_compress   -> pooled keys, pool validity
 *                       -> dsa_compact_pools    -> ascending valid pool ids per sequence
 *                       -> dsa_index_scores     -> [Q, P] scores + candidate flags
 *                          (dsa_compact_index_scores: steps 2 and 3 in one launch)
 *                       -> dsa_topk_pools       -> [Q, select_k] pool ids
 *                       -> dsa_expand_selection -> [Q, out_width] token ids (-1 = none)
 *                       -> dsa_sparse_mla_decode -> [Q, heads, 512] latent-space output
 *
 * Conventions shared by every call
 *  - Pointers named for device data are device pointers (HIP global memory); the caller owns
 *    all of them and the stream. The library never allocates, frees, copies between host
 *    and device, or synchronizes. Kernels are enqueued on `stream` (0 = the null stream).
 *  - Layouts are dense and row-major in the order the brackets give. bf16 is the upper half
 *    of an IEEE binary32 (2 bytes); fp8 is OCP E4M3 ("FN": bias 7, no infinities, max 448),
 *    one byte; ids are int32; masks are one byte, nonzero = true.
 *  - Every argument is checked on the host before anything is launched. On a refusal
 *    nothing is launched, no output is touched, a negative DSA_ERR_* code is returned and
 *    dsa_last_error() describes it. Device-resident values (lengths, ids, positions, token
 *    ids, block-table entries) cannot be checked on the host: the kernels treat any that fall
 *    outside their buffers as absent (a -1 id, a masked token) and never read or write out of
 *    bounds. A failed launch returns DSA_ERR_HIP; faults during execution surface at the
 *    caller's next synchronization.
 *  - Every output element is written by the call (no output relies on a prior fill).
 *  - All calls are safe to record into a HIP graph: they launch kernels only.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status codes */
enum {
    DSA_OK = 0,
    DSA_ERR_NULL_ARG = -1,          /* a required pointer is NULL */
    DSA_ERR_BAD_SIZE = -2,          /* a size or index argument is out of range */
    DSA_ERR_BAD_DTYPE = -3,         /* dtype not accepted by this call */
    /* mod.rs, Glm5NextDsaConfig::validate, its refusals in the page's order */
    DSA_ERR_KPOOL_OR_TOPK_ZERO = -4,
    DSA_ERR_TOPK_NOT_MULTIPLE = -5, /* index_topk must be a multiple of index_kpool */
    DSA_ERR_KPOOL_GT_MAX = -6,      /* index_kpool above DSA_MAX_KPOOL */
    DSA_ERR_KV_LORA_ZERO = -7,
    DSA_ERR_KV_LORA_NOT_512 = -8,   /* the decode kernels are built for a 512-wide latent */
    DSA_ERR_ZERO_HEADS = -9,        /* no MLA heads on this device */
    /* build.rs, absorb_q / absorb_o */
    DSA_ERR_ROPE_UNSUPPORTED = -10, /* absorption is NoPE only */
    DSA_ERR_ELEM_COUNT = -11,       /* a weight's element count does not match the config */
    DSA_ERR_WORKSPACE = -12,        /* workspace missing or smaller than the query says */
    DSA_ERR_HIP = -13,              /* a HIP runtime call failed */
    DSA_ERR_UNSUPPORTED = -14       /* a shape these kernels are not built for */
};

/* Largest index_kpool (mod.rs, KERNEL_MAX_KPOOL) and the latent width (KERNEL_KV_LORA_DIM). */
#define DSA_MAX_KPOOL 8
#define DSA_LATENT_DIM 512
/* Kernel limits of this library: indexer heads per call, index_head_dim values, and the
 * MLA heads handled per 32-head group (more heads run as several groups). */
#define DSA_MAX_INDEX_HEADS 32
/* Most keys dsa_mla_masked_attn takes: its [S] f32 score row sits in 128 KiB of LDS
 * (the pages' kernel: 12,288 in 48 KB, mod.rs MASKED_ATTN_MAX_KEYS). */
#define DSA_MASKED_ATTN_MAX_KEYS 32768

/* Widest token selection (W, token slots per row) dsa_sparse_mla_decode accepts. */
#define DSA_MAX_MLA_WIDTH 32768

typedef enum { DSA_BF16 = 0, DSA_F32 = 1, DSA_FP8_E4M3 = 2 } dsa_dtype;

/* Per-layer DSA geometry (mod.rs, Glm5NextDsaConfig). `heads` is the attention heads this
 * device owns (local_heads); the indexer is replicated, so index_heads is the full count. */
typedef struct {
    int32_t index_heads;
    int32_t index_head_dim;      /* 32, 64 or 128 */
    int32_t index_kpool;         /* pool size, 1..8 */
    int32_t index_topk;          /* token budget, a multiple of index_kpool */
    int32_t always_select_tail;  /* nonzero: out_width gains index_kpool - 1 tail slots */
    int32_t heads;
    int32_t kv_lora_rank;        /* must be 512 */
    int32_t qk_nope_head_dim;
    int32_t qk_rope_head_dim;    /* 0 (NoPE); absorption refuses anything else */
    int32_t v_head_dim;
    int32_t q_lora_rank;
    int32_t hidden;
} dsa_config;

/* Message for the last refusal on the calling thread; valid until that thread's next dsa_*
 * call. Never NULL. */
const char *dsa_last_error(void);

/* Library version string, e.g. "dsa 0.1.0 gfx950". */
const char *dsa_version(void);

/* mod.rs, Glm5NextDsaConfig::validate. Returns DSA_OK or the code of the first failing rule,
 * checked in the page's order: kpool/topk zero, topk not a multiple of kpool, kpool above 8,
 * kv_lora_rank zero, kv_lora_rank not 512, zero heads. */
int dsa_config_validate(const dsa_config *cfg);

/* mod.rs, Glm5NextDsaConfig::select_k: min(index_topk / index_kpool, n_pools).
 * Returns a negative code for an invalid config or n_pools < 0. */
int64_t dsa_select_k(const dsa_config *cfg, int64_t n_pools);

/* mod.rs, Glm5NextDsaConfig::out_width: index_topk (+ index_kpool - 1 with the tail flag). */
int64_t dsa_out_width(const dsa_config *cfg);

/* Whole pools in S token slots when pooling starts at first_key: floor((S - first_key) / kpool),
 * 0 when S <= first_key (mod.rs, "Checkpoint and kernel facts": a trailing partial pool is not
 * a pool). Negative code for kpool <= 0 or negative arguments. */
int64_t dsa_num_pools(int64_t S, int64_t first_key, int64_t kpool);

/* ------------------------------------------------------------------ step 1 */
/* mod.rs, "Shape of the pipeline" and "Checkpoint and kernel facts": pool p of sequence b
 * holds tokens first_key + p*KP + s, s < KP (KP = index_kpool). For every channel d the slot
 * weights are softmax over s of gate[b,t,d] + ape[s,d]; the pooled key is the weighted sum of
 * k[b,t,d], rounded to bf16. A pool is valid only if all KP slots are valid.
 * k, gate: [B, S, D] bf16 (D = index_head_dim)    ape: [KP, D] f32 (build.rs transform 4)
 * valid: [B, S] u8                                 pool_keys: [B, P, D] bf16, pool_valid [B, P]
 * with P = dsa_num_pools(S, first_key, KP). Pooled keys of invalid pools are still written
 * (from whatever the slots hold); only their validity flag says they are unusable. */
int dsa_kpool_compress(const dsa_config *cfg, int B, int S, int first_key, const void *k,
                       const void *gate, const float *ape, const uint8_t *valid, void *pool_keys,
                       uint8_t *pool_valid, hipStream_t stream);

/* The stored fp8 form of fp8 pooled keys and latent rows (the pages keep the selected tokens
 * in fp8 for the serve's decode, mod.rs MASKED_ATTN_MAX_KEYS; the per-row format is this
 * library's reading): per row, scale = amax / 448 with amax the largest |value| of the row
 * (1 for an all-zero row), and each value stored as the OCP e4m3 code nearest to
 * value / scale (ties to even, saturating at +-448); both divisions in IEEE single
 * precision, so the row decodes as code * scale.
 *
 * dsa_kpool_compress with the pooled key stored that way: the bf16 pooled key of
 * dsa_kpool_compress, quantized per pool row. pool_keys: [B, P, D] e4m3 codes (8-byte
 * aligned); pool_key_scales: [B, P] f32; pool_valid as dsa_kpool_compress. D must be a power
 * of two in [8, 512] (DSA_ERR_UNSUPPORTED otherwise). */
int dsa_kpool_compress_fp8(const dsa_config *cfg, int B, int S, int first_key, const void *k,
                           const void *gate, const float *ape, const uint8_t *valid,
                           uint8_t *pool_keys, float *pool_key_scales, uint8_t *pool_valid,
                           hipStream_t stream);

/* Rows of n values quantized as above: src [rows, n] bf16 or f32 (src_dtype, 16-byte
 * aligned), codes [rows, n] e4m3 (8-byte aligned), scales [rows] f32. n must be a multiple
 * of 8 up to 4096 (DSA_ERR_UNSUPPORTED). For the latent cache n = 512. */
int dsa_quantize_rows_fp8(int64_t rows, int n, const void *src, dsa_dtype src_dtype, uint8_t *codes,
                          float *scales, hipStream_t stream);

/* ------------------------------------------------------------------ decode-time upkeep */
/* The per-step maintenance of the indexer cache that comes before the selection chain in a
 * decode step (one new token per sequence). The pages name these kernels in mod.rs,
 * Glm5NextDsaKernels.
 *
 * k_norm: indexer.k_norm is a LayerNorm with a bias (not an RMSNorm), applied in place:
 * per row of D values, y = (x - mean) / sqrt(var + eps) * weight + bias with the biased
 * variance, f32 arithmetic, bf16 out. x: [rows, D] bf16 (in place, 16-byte aligned);
 * weight, bias: [D] bf16. D must be 8 times a power of two, at most 512. */
int dsa_k_norm(int64_t rows, int D, void *x, const void *weight, const void *bias, float eps,
               hipStream_t stream);

/* indexer_store: copies each sequence's staged indexer row -- the new token's (normalized)
 * key and its gate values -- to the device-side position pos[b] and marks that slot valid.
 * A position outside [0, S) stores nothing. pos: [B] i32 (device); k_row, gate_row: [B, D]
 * bf16; k_cache, gate_cache: [B, S, D] bf16; valid: [B, S] u8. D a multiple of 8. */
int dsa_indexer_store(int B, int S, int D, const int32_t *pos, const void *k_row, const void *gate_row,
                      void *k_cache, void *gate_cache, uint8_t *valid, hipStream_t stream);

/* write_geom: the selector geometry from the live lengths, on the device (so a captured graph
 * replays over the live context): one decode row per sequence, row_seq[b] = b and
 * row_pos[b] = seq_len[b] - 1. seq_len, row_seq, row_pos: [B] i32. */
int dsa_write_geom(int B, const int32_t *seq_len, int32_t *row_seq, int32_t *row_pos, hipStream_t stream);

/* pool_append: the pool that the token at pos[b] completes (mod.rs, "Checkpoint and kernel
 * facts": pooling starts at first_key; a pool counts only when all its slots are valid). When
 * pos >= first_key, (pos - first_key + 1) % KP == 0 and p = (pos - first_key + 1)/KP - 1 < P,
 * pool p's key and validity are computed exactly as dsa_kpool_compress (bf16 keys,
 * pool_key_scales NULL) or dsa_kpool_compress_fp8 (fp8 codes, pool_key_scales [B, P]) computes
 * them, and a valid p is appended to the compacted list of dsa_compact_pools
 * (ids[b, n_valid[b]] = p, n_valid[b] += 1) unless the list already ends at p or beyond, so
 * a repeated call changes nothing. Other positions change nothing. Storing every token this
 * way keeps pool_keys, pool_valid, ids and n_valid equal to the batch calls. Arguments as
 * dsa_kpool_compress and dsa_compact_pools; pos: [B] i32 (device). D a power of two in
 * [8, 512]. */
int dsa_pool_append(const dsa_config *cfg, int B, int S, int first_key, const int32_t *pos,
                    const void *k, const void *gate, const float *ape, const uint8_t *valid,
                    void *pool_keys, float *pool_key_scales, uint8_t *pool_valid, int32_t *ids,
                    int32_t *n_valid, hipStream_t stream);

/* ------------------------------------------------------------------ step 2 */
/* mod.rs names dsa_compact_pools between pooling and scoring. Stable compaction per
 * sequence: ids[b, 0..n_valid[b]) are the valid pool indices in ascending order, the rest of
 * the row is -1. pool_valid: [B, P] u8; ids: [B, P] i32; n_valid: [B] i32. */
int dsa_compact_pools(int B, int P, const uint8_t *pool_valid, int32_t *ids, int32_t *n_valid,
                      hipStream_t stream);

/* ------------------------------------------------------------------ step 3 */
/* tp.rs, "Why the indexer is replicated": score[r, p] = sum over indexer heads h of
 * w[r, h] * relu(scale * q[r, h, :] . key[b, p, :]), b = row_seq[r]; build.rs transform 2:
 * w already carries index_heads^-0.5, this call does not apply it. For fp8 keys the dot is
 * multiplied by key_scales[b, p]. Pool p is a candidate for row r when it appears in
 * ids[b, 0..n_valid[b]) and its last token first_key + (p+1)*KP - 1 <= row_pos[r].
 * Candidates get their f32 score (-0 written as +0) and cand = 1; every other slot gets
 * -inf and cand = 0.
 * q: [Q, Hi, D] bf16    w: [Q, Hi] f32    row_seq, row_pos: [Q] i32
 * keys: [B, P, D] bf16 or fp8 (key_dtype)   key_scales: [B, P] f32 (fp8 only, else NULL)
 * ids: [B, P] i32, n_valid: [B] i32 (dsa_compact_pools output)
 * scores: [Q, P] f32    cand: [Q, P] u8 */
int dsa_index_scores(const dsa_config *cfg, int Q, int B, int P, int first_key, float scale,
                     const void *q, const float *w, const int32_t *row_seq,
                     const int32_t *row_pos, const void *keys, dsa_dtype key_dtype,
                     const float *key_scales, const int32_t *ids, const int32_t *n_valid,
                     float *scores, uint8_t *cand, hipStream_t stream);

/* ------------------------------------------------------------------ steps 2 and 3 fused */
/* mod.rs, "Shape of the pipeline" (dsa_compact_pools, then dsa_index_scores), in one launch:
 * pool p is a candidate for row r when pool_valid[b, p] != 0 (b = row_seq[r]) and its last
 * token first_key + (p+1)*KP - 1 <= row_pos[r]. scores and cand are exactly those of
 * dsa_compact_pools followed by dsa_index_scores on the same flags; the compacted id list is
 * never materialised (each block reads the flags of its own pool range and loads keys only for
 * candidates, which is the read the compaction saves).
 * pool_valid: [B, P] u8 (dsa_kpool_compress output); the other arguments as dsa_index_scores. */
int dsa_compact_index_scores(const dsa_config *cfg, int Q, int B, int P, int first_key,
                             float scale, const void *q, const float *w, const int32_t *row_seq,
                             const int32_t *row_pos, const void *keys, dsa_dtype key_dtype,
                             const float *key_scales, const uint8_t *pool_valid, float *scores,
                             uint8_t *cand, hipStream_t stream);

/* ------------------------------------------------------------------ step 4 */
/* mod.rs, "Shape of the pipeline": [Q, select_k] pool ids. Per row, the Kw candidates that
 * rank first by (score descending, pool index ascending) are written in ascending pool order,
 * then -1 up to Kw. Equal scores (-0 == +0) go to the lower pool index, the tie rule tp.rs
 * shows is needed for a stable selection. Kw = dsa_select_k(cfg, P).
 * scores: [Q, P] f32; cand: [Q, P] u8; sel: [Q, Kw] i32. Scores must not be NaN.
 * ws: device workspace of dsa_topk_workspace(cfg, Q, P) bytes (16-byte aligned), or NULL with
 * ws_bytes 0. Given it, few long rows (at most 64 rows of several 8,192-pool segments) are
 * selected in two launches: each segment's best Kw first (one block per row and segment),
 * then the row's best Kw among those; without it, or when too small, one block per row selects
 * from the whole row. Both give the same sel. */
size_t dsa_topk_workspace(const dsa_config *cfg, int Q, int P);
/* Alias of dsa_topk_workspace named after dsa_topk_pools: identical result. */
size_t dsa_topk_pools_workspace(const dsa_config *cfg, int Q, int P);
int dsa_topk_pools(const dsa_config *cfg, int Q, int P, const float *scores, const uint8_t *cand,
                   int32_t *sel, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ step 5 */
/* mod.rs, "Shape of the pipeline" and "Checkpoint and kernel facts": token ids of the selected
 * pools, -1 where there is none. Slot i*KP + s holds first_key + p*KP + s for sel[r, i] = p
 * (p outside [0, P) counts as -1). With always_select_tail, slots index_topk .. index_topk+KP-2
 * hold the tokens after the last whole pool up to row_pos[r], each only if valid.
 * sel: [Q, Kw] i32 (Kw*KP <= index_topk); row_seq, row_pos: [Q] i32; valid: [B, S] u8 (only
 * read with the tail flag; may be NULL otherwise); token_ids: [Q, dsa_out_width(cfg)] i32. */
int dsa_expand_selection(const dsa_config *cfg, int Q, int Kw, int B, int S, int first_key,
                         const int32_t *sel, const int32_t *row_seq, const int32_t *row_pos,
                         const uint8_t *valid, int32_t *token_ids, hipStream_t stream);

/* ------------------------------------------------------------------ steps 4 and 5 fused */
/* mod.rs, "Shape of the pipeline": the selection and its expansion in one launch. Writes the
 * same sel [Q, Kw] (Kw = dsa_select_k(cfg, P)) as dsa_topk_pools and the same token_ids
 * [Q, dsa_out_width(cfg)] as dsa_expand_selection given that sel; the selection is not read
 * back from memory. P must not exceed dsa_num_pools(S, first_key, kpool) (DSA_ERR_BAD_SIZE).
 * Arguments as in the two calls; scores, cand and sel may be NULL only when Kw = 0. The
 * workspace as dsa_topk_pools's (dsa_topk_workspace), or NULL. */
int dsa_topk_expand(const dsa_config *cfg, int Q, int P, const float *scores, const uint8_t *cand,
                    int B, int S, int first_key, const int32_t *row_seq, const int32_t *row_pos,
                    const uint8_t *valid, int32_t *sel, int32_t *token_ids, void *ws,
                    size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ step 6 */
/* build.rs, "The transforms" 1 and 3, and mod.rs (NoPE, 512-wide latent, attention restricted
 * to the selected tokens, paged reads through a block table): for row r and head h, over the
 * row's token ids t >= 0, with v_t the 512-wide latent row of token t of sequence
 * b = row_seq[r]: logit_t = sm_scale * q_abs[r,h,:] . v_t, out[r,h,:] = sum_t softmax_t * v_t.
 * Keys and values are the same latent rows. lse[r,h] = log sum exp(logit) (natural log).
 * A row with no token gives out = 0 and lse = -inf.
 * q_abs: [Q, heads, 512] bf16; token_ids: [Q, W] i32; row_seq: [Q] i32 in [0, B).
 * kv: [kv_rows, 512] bf16 or fp8 (kv_dtype); kv_scales: [kv_rows] f32 for fp8 (the latent
 * row is e4m3 * scale), else NULL. Row of token t: contiguous (block_table == NULL)
 * b*S + t; paged: block_table[b*max_blocks + t/block_size]*block_size + t%block_size with
 * block_table [B, max_blocks] i32. Token ids at or past S (when S > 0), blocks mapped to a
 * negative entry, and rows outside [0, kv_rows) are skipped like -1. A contiguous latent
 * needs S > 0 (DSA_ERR_BAD_SIZE otherwise, when W > 0); paged, S = 0 sets no bound.
 * out: [Q, heads, 512] f32; lse: [Q, heads] f32 or NULL.
 * W above DSA_MAX_MLA_WIDTH or kv_rows above 2^31 - 1 is refused with DSA_ERR_UNSUPPORTED.
 * ws: device workspace of at least dsa_sparse_mla_decode_workspace(cfg, Q, W) bytes
 * (may be NULL when that is 0). */
size_t dsa_sparse_mla_decode_workspace(const dsa_config *cfg, int Q, int W);
int dsa_sparse_mla_decode(const dsa_config *cfg, int Q, int W, int B, float sm_scale,
                          const void *q_abs, const int32_t *token_ids, const int32_t *row_seq,
                          const void *kv, dsa_dtype kv_dtype, const float *kv_scales,
                          int64_t kv_rows, int S, const int32_t *block_table, int max_blocks,
                          int block_size, float *out, float *lse, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): dsa_sparse_mla_decode without the workspace
 * argument. The split partials go to a fixed 16 MiB device array inside the library
 * (DSA_MLA_NOALLOC_SCRATCH_BYTES), one copy per GPU, held until the process ends and looked
 * up on the first call on each device; nothing is allocated, and the result is bit-identical
 * to dsa_sparse_mla_decode's. Arguments, layouts and refusals are those of
 * dsa_sparse_mla_decode; a call whose workspace query exceeds the scratch size is refused
 * with DSA_ERR_WORKSPACE before anything is launched. Every call on one GPU shares that GPU's
 * scratch, which keeps the last call's partials: calls that overlap on one GPU (different
 * streams, or threads) race and must be ordered by the caller. */
#define DSA_MLA_NOALLOC_SCRATCH_BYTES (16u << 20)
int dsa_sparse_mla_decode_noalloc(const dsa_config *cfg, int Q, int W, int B, float sm_scale,
                                  const void *q_abs, const int32_t *token_ids,
                                  const int32_t *row_seq, const void *kv, dsa_dtype kv_dtype,
                                  const float *kv_scales, int64_t kv_rows, int S,
                                  const int32_t *block_table, int max_blocks, int block_size,
                                  float *out, float *lse, hipStream_t stream);

/* ------------------------------------------------------------------ dense masked cross-check */
/* mod.rs, Glm5NextDsaKernels::{topk_to_mask, mla_masked_attn} and MASKED_ATTN_MAX_KEYS: the
 * selection as a token mask, and a dense attention over every masked token that stages the
 * whole [S] score row; a second route to dsa_sparse_mla_decode's result, used to check it.
 *
 * topk_to_mask: mask[r, t] = 1 when some slot of token_ids[r] holds t (0 <= t < S), else 0;
 * every element written. token_ids: [Q, W] i32; mask: [Q, S] u8. */
int dsa_topk_to_mask(int Q, int W, int S, const int32_t *token_ids, uint8_t *mask,
                     hipStream_t stream);

/* mla_masked_attn: for row r and head h, over every t < S with mask[r, t] = 1 (ascending),
 * logit_t = sm_scale * q_abs[r,h,:] . v_t and out[r,h,:] = sum_t softmax_t v_t,
 * lse[r,h] = log sum exp(logit); latent rows, dtypes, paging and skipped rows exactly as
 * dsa_sparse_mla_decode (S is also the contiguous stride). A row without a token gives
 * out = 0, lse = -inf. S above DSA_MASKED_ATTN_MAX_KEYS is refused (DSA_ERR_UNSUPPORTED).
 * q_abs: [Q, heads, 512] bf16; mask: [Q, S] u8; out: [Q, heads, 512] f32; lse: [Q, heads]
 * f32 or NULL. One block per (row, head), f32 arithmetic: a check, not the decode path. */
int dsa_mla_masked_attn(const dsa_config *cfg, int Q, int S, int B, float sm_scale,
                        const void *q_abs, const uint8_t *mask, const int32_t *row_seq,
                        const void *kv, dsa_dtype kv_dtype, const float *kv_scales,
                        int64_t kv_rows, const int32_t *block_table, int max_blocks,
                        int block_size, float *out, float *lse, hipStream_t stream);

/* ------------------------------------------------------------------ host weight prep */
/* build.rs, absorb_q / absorb_q_rows (host memory, f32): q_absorb[h*kvl + c][k] =
 * sum over r < nope of kv_b[h*(nope+vd) + r][c] * q_b[h*nope + r][k], r ascending, each
 * output element accumulated in one thread with a separate multiply and add, so the result
 * does not depend on the thread count.
 * q_b: [full_heads*(nope+rope), q_lora_rank]; kv_b: [full_heads*(nope+vd), kv_lora_rank];
 * out: [full_heads*kv_lora_rank, q_lora_rank]. threads: > 0 uses that many; 0 reads the
 * environment variable DSA_ABSORB_THREADS (a positive integer) and otherwise uses the
 * hardware concurrency; the count is clamped to 1..rows. Refuses a nonzero rope width and
 * element counts that do not match (DSA_ERR_ELEM_COUNT). */
int dsa_absorb_q(const dsa_config *cfg, const float *q_b, size_t q_b_len, const float *kv_b,
                 size_t kv_b_len, int full_heads, int threads, float *out, size_t out_len);

/* build.rs, absorb_o (host memory, f32): o_absorb[i][h*kvl + c] =
 * sum over r < vd of o_local[i][h*vd + r] * kv_b_local[h*(nope+vd) + nope + r][c],
 * r ascending, per element in one thread. o_local: [hidden, local_heads*vd];
 * kv_b_local: [local_heads*(nope+vd), kvl]; out: [hidden, local_heads*kvl].
 * threads as for dsa_absorb_q (clamped to 1..hidden). */
int dsa_absorb_o(const dsa_config *cfg, const float *o_local, size_t o_len,
                 const float *kv_b_local, size_t kv_len, int local_heads, int threads,
                 float *out, size_t out_len);

/* build.rs, up_bf16: host f32 -> bf16 by round to nearest, ties to even (NaN stays NaN). */
void dsa_f32_to_bf16_rne(const float *src, uint16_t *dst, size_t n);

/* ------------------------------------------------------------------ measurement only */
/* Not a step of the method: reads every byte of buf (device memory, 16-byte aligned, bytes a
 * multiple of 16) once with plain streaming 16-byte loads and XORs the words into *sink (device,
 * not cleared). The rate it reaches is the achievable HBM read bandwidth that the decode
 * kernels' bandwidth is reported against, beside the nominal peak. */
int dsa_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Not a step of the method: launches a kernel of `blocks` (1 .. 65535) blocks of 64 threads
 * that does nothing. A graph of many such launches, replayed, gives the gap between dependent
 * launches on the stream. DSA_ERR_BAD_SIZE for blocks out of range. */
int dsa_empty_launch(int blocks, hipStream_t stream);

/* Not a step of the method: the matrix units' dense rate. Each of the `blocks` (1 .. 65535)
 * blocks has 4 waves; each wave runs `iters` (even, >= 2) rounds of 4 independent MFMAs of one shape:
 * kind 0 = v_mfma_f32_32x32x16_bf16, 1 = v_mfma_f32_16x16x32_bf16, 2 =
 * v_mfma_scale_f32_16x16x128_f8f6f4 with e4m3 operands. One launch performs
 * blocks * 4 * iters * 4 * 2*M*N*K floating-point operations (M*N*K = 16384 for kinds 0 and 1,
 * 32768 for kind 2). out (device, blocks * 256 floats) receives one sum per thread so the work
 * cannot be dropped. DSA_ERR_BAD_SIZE for an argument out of range, DSA_ERR_NULL_ARG for out. */
int dsa_mfma_rate(int kind, int blocks, int iters, float *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */

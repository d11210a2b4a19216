/*
 * dsa_oracle.c -- CPU oracle for the pooled-key DSA indexer and sparse NoPE-MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the package smoke check and the CPU-baseline leg of
 * the benchmark load this file's shared object; the GPU library never does, and this file
 * shares no source, header, table or helper with it.
 *
 * Plain and slow on purpose: one loop nest per definition, every floating-point step in
 * double, results rounded once to the output type (f32, or bf16 by round-to-nearest-even of
 * the f32 value, the rounding the upload path of build.rs uses). The absorb transforms are
 * the exception: they follow the f32 arithmetic and loop order that build.rs gives for them.
 * Built with -O2 -ffp-contract=off, no fast-math. The only parallelism is an OpenMP loop
 * over independent output rows, which changes no arithmetic.
 *
 * Sources (documentation pages of metrale_model_arch::glm5next_dsa):
 *   mod.rs   -- module doc "Shape of the pipeline" and "Checkpoint and kernel facts",
 *               Glm5NextDsaConfig::{select_k, out_width, validate}
 *   build.rs -- module doc "The transforms", absorb_q_rows, absorb_q, absorb_o
 *   tp.rs    -- module doc "Why the indexer is replicated" (the index score rule)
 * Where the pages leave a step open, the reading taken is stated at the function.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- number formats */

/* bf16 is the top half of an IEEE binary32. */
static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* binary32 -> bf16, round to nearest, ties to even (NaN kept quiet). */
static uint16_t bf16_from_float(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

/* OCP 8-bit floating point, E4M3 ("FN": no infinities, S.1111.111 is NaN):
 * sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent field 0 is
 * subnormal, value mantissa/8 * 2^-6. */
static double e4m3_value(uint8_t c) {
    int sign = (c >> 7) & 1, ex = (c >> 3) & 15, man = c & 7;
    double v;
    if (ex == 15 && man == 7) return NAN;
    if (ex == 0) v = ldexp((double)man / 8.0, -6);
    else v = ldexp(1.0 + (double)man / 8.0, ex - 7);
    return sign ? -v : v;
}

/* f64 result rounded once to f32; a zero of either sign comes back as +0. */
static float to_f32_canonical(double x) {
    float f = (float)x;
    if (f == 0.0f) f = 0.0f;
    return f;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

double orc_bf16_value(uint16_t h) { return bf16_value(h); }
double orc_e4m3_value(uint8_t c) { return e4m3_value(c); }
uint16_t orc_bf16_from_float(float f) { return bf16_from_float(f); }

/* ---------------------------------------------------------------- geometry + validation */

/* Glm5NextDsaConfig::select_k (mod.rs): pools selected per query, the pool budget
 * index_topk / index_kpool capped by the number of pools. */
long orc_select_k(long index_topk, long index_kpool, long n_pools) {
    long k = index_topk / index_kpool;
    return k < n_pools ? k : n_pools;
}

/* Glm5NextDsaConfig::out_width (mod.rs): index row width is index_topk, with
 * index_kpool - 1 extra tail slots when always_select_tail is set. */
long orc_out_width(long index_topk, long index_kpool, int always_select_tail) {
    return index_topk + (always_select_tail ? index_kpool - 1 : 0);
}

/* Number of whole pools in S token slots when pooling starts at first_key (mod.rs,
 * "Checkpoint and kernel facts": pooling starts at first_key and a trailing partial pool is
 * not a pool). With first_key = 0 this is tp.rs's seq / kpool. */
long orc_num_pools(long S, long first_key, long kpool) {
    if (kpool <= 0 || S <= first_key) return 0;
    return (S - first_key) / kpool;
}

/* Glm5NextDsaConfig::validate (mod.rs), its six refusals in the page's order.
 * Returns 0 when the config is accepted, else the 1-based number of the first failing
 * rule: 1 kpool or topk zero, 2 topk not a multiple of kpool, 3 kpool above the 8-slot
 * kernel bound, 4 kv_lora_rank zero, 5 kv_lora_rank not the 512 the decode kernel is built
 * for, 6 no attention heads on this rank. */
int orc_validate(long index_kpool, long index_topk, long kv_lora_rank, long local_heads) {
    if (index_kpool == 0 || index_topk == 0) return 1;
    if (index_topk % index_kpool != 0) return 2;
    if (index_kpool > 8) return 3;
    if (kv_lora_rank == 0) return 4;
    if (kv_lora_rank != 512) return 5;
    if (local_heads == 0) return 6;
    return 0;
}

/* ---------------------------------------------------------------- fp8 writers */

/* binary32 -> OCP E4M3 ("FN") code: the representable value nearest to x, ties to the code
 * with an even mantissa, magnitudes beyond the largest normal (448) saturating to it; the
 * sign is kept (so a negative value that rounds to zero gives 0x80). Found by binary search
 * over the 127 non-negative finite values of e4m3_value, compared in double. */
static uint8_t e4m3_from_float(float x) {
    double a = fabs((double)x);
    uint8_t sign = signbit(x) ? 0x80u : 0x00u;
    int lo = 0, hi = 0x7e; /* codes 0 .. 0x7e are the non-negative finite values, ascending */
    if (a >= e4m3_value(0x7e)) return (uint8_t)(sign | 0x7e);
    while (hi - lo > 1) { /* invariant: value(lo) <= a < value(hi) */
        int mid = (lo + hi) / 2;
        if (e4m3_value((uint8_t)mid) <= a) lo = mid;
        else hi = mid;
    }
    double dl = a - e4m3_value((uint8_t)lo), dh = e4m3_value((uint8_t)hi) - a;
    int code = dl < dh ? lo : (dh < dl ? hi : ((lo & 1) ? hi : lo));
    return (uint8_t)(sign | code);
}

uint8_t orc_e4m3_from_float(float x) { return e4m3_from_float(x); }

/* Per-row fp8 quantizer (the reading of the stored fp8 format: per row scale
 * s = amax / 448 with amax the largest |x| of the row, s = 1 for an all-zero row; each value
 * stored as e4m3(x / s), so that the row is code * s). s and x / s are single-precision
 * divisions, as the stored scale is f32. Layouts: x [rows, n] f32 values; codes [rows, n];
 * scales [rows]. */
void orc_quantize_rows(long rows, int n, const float *x, uint8_t *codes, float *scales) {
    for (long r = 0; r < rows; ++r) {
        float amax = 0.0f;
        for (int i = 0; i < n; ++i) {
            float a = fabsf(x[r * n + i]);
            if (a > amax) amax = a;
        }
        volatile float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        scales[r] = s;
        for (int i = 0; i < n; ++i) {
            volatile float q = x[r * n + i] / s;
            codes[r * n + i] = e4m3_from_float(q);
        }
    }
}

/* ---------------------------------------------------------------- step 1: kpool_compress */

/* mod.rs, "Shape of the pipeline" (k, gate, valid, ape -> pool keys / indices / valid) and
 * "Checkpoint and kernel facts" (softmax over the pool-slot axis, per channel; pooling starts
 * at first_key; a pool counts only if all index_kpool slots are valid). build.rs transform 4:
 * ape is f32.
 * Reading: pool p of sequence b covers tokens t_s = first_key + p*KP + s, s < KP. For each
 * channel d the slot weights are softmax_s(gate[b,t_s,d] + ape[s,d]) and the pooled key is
 * the weighted sum of k[b,t_s,d]; it is stored as bf16. The pool index p itself is the pool's
 * identity (its first token is first_key + p*KP), so no separate index array is written.
 * Layouts: k, gate [B,S,D] bf16; ape [KP,D] f32; valid [B,S] u8;
 * pool_keys [B,P,D] bf16; pool_valid [B,P] u8, with P = orc_num_pools(S, first_key, KP). */
static void compress_pool(long b, long p, long P, int S, int D, int KP, int first_key,
                          const uint16_t *k, const uint16_t *gate, const float *ape,
                          const uint8_t *valid, uint16_t *pool_keys, uint8_t *pool_valid);

void orc_kpool_compress(int B, int S, int D, int KP, int first_key,
                        const uint16_t *k, const uint16_t *gate, const float *ape,
                        const uint8_t *valid, uint16_t *pool_keys, uint8_t *pool_valid) {
    long P = orc_num_pools(S, first_key, KP);
    long bp;
#pragma omp parallel for schedule(static)
    for (bp = 0; bp < (long)B * P; ++bp)
        compress_pool(bp / P, bp % P, P, S, D, KP, first_key, k, gate, ape, valid, pool_keys,
                      pool_valid);
}

/* Pool p of sequence b (the body of orc_kpool_compress). */
static void compress_pool(long b, long p, long P, int S, int D, int KP, int first_key,
                          const uint16_t *k, const uint16_t *gate, const float *ape,
                          const uint8_t *valid, uint16_t *pool_keys, uint8_t *pool_valid) {
    {
        long t0 = (long)first_key + p * KP;
        int ok = 1;
        for (int s = 0; s < KP; ++s)
            if (!valid[b * S + t0 + s]) ok = 0;
        pool_valid[b * P + p] = (uint8_t)ok;
        for (int d = 0; d < D; ++d) {
            double logit[64], mx = -INFINITY, den = 0.0, acc = 0.0;
            for (int s = 0; s < KP; ++s) {
                logit[s] = bf16_value(gate[(b * S + t0 + s) * D + d]) + (double)ape[s * D + d];
                if (logit[s] > mx) mx = logit[s];
            }
            for (int s = 0; s < KP; ++s) den += exp(logit[s] - mx);
            for (int s = 0; s < KP; ++s)
                acc += (exp(logit[s] - mx) / den) * bf16_value(k[(b * S + t0 + s) * D + d]);
            pool_keys[(b * P + p) * D + d] = bf16_from_float((float)acc);
        }
    }
}

/* ---------------------------------------------------------------- step 2: compact_pools */

/* mod.rs names dsa_compact_pools between pooling and scoring and says no more.
 * Reading: a stable compaction. ids[b, 0..n_valid[b]) are the valid pool indices of sequence
 * b in ascending order, the remaining entries are -1; n_valid[b] is their count.
 * Layouts: pool_valid [B,P] u8; ids [B,P] i32; n_valid [B] i32. */
void orc_compact_pools(int B, int P, const uint8_t *pool_valid, int32_t *ids, int32_t *n_valid) {
    for (long b = 0; b < B; ++b) {
        int32_t n = 0;
        for (long p = 0; p < P; ++p)
            if (pool_valid[b * P + p]) ids[b * P + n++] = (int32_t)p;
        n_valid[b] = n;
        for (long j = n; j < P; ++j) ids[b * P + j] = -1;
    }
}

/* ---------------------------------------------------------------- step 3: index_scores */

/* tp.rs, "Why the indexer is replicated": a pool's score adds weights[h] * relu(scale * dot)
 * over the indexer heads, giving [q_rows, n_pools] scores. build.rs transform 2: the
 * index_heads^-0.5 factor is already folded into the weights, the scorer does not apply it.
 * mod.rs, "Shape of the pipeline": the output is the score array plus candidate validity.
 * Readings: w is given per query row and head ([Q,Hi] f32, already scaled). The dot is
 * q[r,h,:] . key[b,p,:] with b = row_seq[r]; for fp8 keys the dot of the decoded e4m3 values
 * is multiplied by the pool's f32 scale. A pool is a candidate for row r when it is listed in
 * the compacted valid list of its sequence and its last token first_key + (p+1)*KP - 1 is at
 * or before the row's position row_pos[r] (decode rows sit at the last valid token, prefill
 * rows are causal). Heads are summed in ascending order in double; the f32 result has
 * -0 turned into +0. Non-candidate slots get -inf and cand = 0.
 * Layouts: q [Q,Hi,D] bf16; w [Q,Hi] f32; row_seq/row_pos [Q] i32; keys [B,P,D] bf16 or e4m3
 * (key_fp8 = 1) with key_scales [B,P] f32; ids [B,P], n_valid [B] i32;
 * scores [Q,P] f32; cand [Q,P] u8. */
void orc_index_scores(int Q, int B, int P, int Hi, int D, int KP, int first_key, double scale,
                      const uint16_t *q, const float *w, const int32_t *row_seq,
                      const int32_t *row_pos, const void *keys, int key_fp8,
                      const float *key_scales, const int32_t *ids, const int32_t *n_valid,
                      float *scores, uint8_t *cand) {
    (void)B;
    long r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < Q; ++r) {
        long b = row_seq[r], pos = row_pos[r];
        for (long p = 0; p < P; ++p) {
            scores[r * P + p] = -INFINITY;
            cand[r * P + p] = 0;
        }
        for (long j = 0; j < n_valid[b]; ++j) {
            long p = ids[b * P + j];
            long last_token = (long)first_key + (p + 1) * KP - 1;
            if (last_token > pos) continue;
            double key_scale = key_fp8 ? (double)key_scales[b * P + p] : 1.0;
            double total = 0.0;
            for (int h = 0; h < Hi; ++h) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) {
                    double qv = bf16_value(q[(r * Hi + h) * D + d]);
                    double kv = key_fp8 ? e4m3_value(((const uint8_t *)keys)[(b * P + p) * D + d])
                                        : bf16_value(((const uint16_t *)keys)[(b * P + p) * D + d]);
                    dot += qv * kv;
                }
                double x = scale * (key_scale * dot);
                total += (double)w[r * Hi + h] * (x > 0.0 ? x : 0.0);
            }
            scores[r * P + p] = to_f32_canonical(total);
            cand[r * P + p] = 1;
        }
    }
}

/* ---------------------------------------------------------------- step 4: topk_pools */

typedef struct { float score; int32_t pool; } scored_pool;

/* Ranking key: higher score first; among equal scores the lower pool index first. */
static int by_score_then_pool(const void *a, const void *b) {
    const scored_pool *x = (const scored_pool *)a, *y = (const scored_pool *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->pool > y->pool) - (x->pool < y->pool);
}

static int by_pool(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* mod.rs, "Shape of the pipeline": topk_pools turns the scores into [Q, select_k] pool ids;
 * select_k = min(index_topk / index_kpool, n_pools).
 * Readings: the Kw best candidates by (score descending, pool index ascending) are chosen;
 * equal scores go to the lower pool index (tp.rs warns that ties at the cutoff are order
 * sensitive, so the rule is fixed). The chosen ids are written in ascending pool order; a row
 * with fewer than Kw candidates is padded with -1. Scores compare as floats, so -0 == +0.
 * Layouts: scores [Q,P] f32; cand [Q,P] u8; sel [Q,Kw] i32. */
void orc_topk_pools(int Q, int P, int Kw, const float *scores, const uint8_t *cand, int32_t *sel) {
    long r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < Q; ++r) {
        scored_pool *list = (scored_pool *)malloc(sizeof(scored_pool) * (size_t)(P > 0 ? P : 1));
        int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * (size_t)(Kw > 0 ? Kw : 1));
        long n = 0;
        for (long p = 0; p < P; ++p)
            if (cand[r * P + p]) {
                list[n].score = scores[r * P + p];
                list[n].pool = (int32_t)p;
                ++n;
            }
        qsort(list, (size_t)n, sizeof(scored_pool), by_score_then_pool);
        long take = n < Kw ? n : Kw;
        for (long i = 0; i < take; ++i) chosen[i] = list[i].pool;
        qsort(chosen, (size_t)take, sizeof(int32_t), by_pool);
        for (long i = 0; i < Kw; ++i) sel[r * Kw + i] = i < take ? chosen[i] : -1;
        free(list);
        free(chosen);
    }
}

/* ---------------------------------------------------------------- step 5: expand_selection */

/* mod.rs, "Shape of the pipeline" ([Q, out_width] token ids, -1 = invalid) and "Checkpoint
 * and kernel facts" (-1 goes over the whole row before any index is stored, so every slot is
 * written); Glm5NextDsaConfig::out_width for the row width.
 * Readings: selected pool i (sel[r,i] = p >= 0) fills slots i*KP .. i*KP+KP-1 with tokens
 * first_key + p*KP + s. With always_select_tail the tokens after the last whole pool up to and
 * including the row's position, t in [tail_start, pos] with
 * tail_start = first_key + floor((pos + 1 - first_key) / KP) * KP, go to slots
 * index_topk + (t - tail_start); a tail token that is not valid stays -1.
 * Layouts: sel [Q,Kw] i32; row_seq/row_pos [Q] i32; valid [B,S] u8; token_ids [Q,W] i32. */
void orc_expand_selection(int Q, int Kw, int KP, int index_topk, int always_select_tail, int S,
                          int first_key, const int32_t *sel, const int32_t *row_seq,
                          const int32_t *row_pos, const uint8_t *valid, int32_t *token_ids) {
    long W = orc_out_width(index_topk, KP, always_select_tail);
    for (long r = 0; r < Q; ++r) {
        int32_t *row = token_ids + r * W;
        for (long i = 0; i < W; ++i) row[i] = -1;
        for (long i = 0; i < Kw; ++i) {
            long p = sel[r * Kw + i];
            if (p < 0) continue;
            for (long s = 0; s < KP; ++s) row[i * KP + s] = (int32_t)(first_key + p * KP + s);
        }
        if (always_select_tail) {
            long b = row_seq[r], pos = row_pos[r];
            if (pos + 1 > first_key) {
                long tail_start = first_key + ((pos + 1 - first_key) / KP) * KP;
                for (long t = tail_start; t <= pos; ++t)
                    if (t < S && valid[b * S + t]) row[index_topk + (t - tail_start)] = (int32_t)t;
            }
        }
    }
}

/* ---------------------------------------------------------------- step 6: sparse MLA decode */

/* build.rs, "The transforms" (1 and 3): the query is absorbed into the kv_lora_rank-wide latent
 * space and the decode output is [local_heads, kv_lora_rank] in that space; mod.rs: NoPE (no
 * rope section), latent width 512, attention restricted to the expanded tokens; the serve
 * decode reads the selected tokens through a block table.
 * Readings: for row r and head h, over the row's token ids t >= 0 (in slot order), with v_t
 * the latent row of token t of sequence b = row_seq[r] (bf16, or e4m3 times the row's f32
 * scale): logit_t = sm * (q_abs[r,h,:] . v_t), out[r,h,:] = sum_t softmax(logit)_t * v_t;
 * keys and values are the same latent rows. lse = max + log(sum exp(logit - max)). A row with
 * no token gives out = 0 and lse = -inf.
 * Latent row address: contiguous, b*S + t; paged (block_table != NULL),
 * block_table[b*max_blocks + t/block_size]*block_size + t%block_size. kv_scales (fp8 only)
 * is indexed by the same row number.
 * Layouts: q_abs [Q,H,C] bf16; token_ids [Q,W] i32; row_seq [Q] i32; kv [rows,C] bf16/e4m3;
 * out [Q,H,C] f32; lse [Q,H] f32 (may be NULL). */
void orc_sparse_mla(int Q, int H, int C, int W, double sm, const uint16_t *q_abs,
                    const int32_t *token_ids, const int32_t *row_seq, const void *kv, int kv_fp8,
                    const float *kv_scales, int S, const int32_t *block_table, int max_blocks,
                    int block_size, float *out, float *lse) {
    long r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < Q; ++r) {
        long b = row_seq[r];
        long *rows = (long *)malloc(sizeof(long) * (size_t)(W > 0 ? W : 1));
        double *logit = (double *)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
        double *v = (double *)malloc(sizeof(double) * (size_t)C);
        long n = 0;
        for (long i = 0; i < W; ++i) {
            long t = token_ids[r * W + i];
            if (t < 0) continue;
            long row = block_table ? (long)block_table[b * max_blocks + t / block_size] * block_size +
                                         t % block_size
                                   : b * (long)S + t;
            rows[n++] = row;
        }
        for (long h = 0; h < H; ++h) {
            const uint16_t *qh = q_abs + (r * H + h) * C;
            float *oh = out + (r * H + h) * C;
            double mx = -INFINITY, den = 0.0;
            for (long i = 0; i < n; ++i) {
                double dot = 0.0;
                for (long c = 0; c < C; ++c) {
                    double vc = kv_fp8 ? e4m3_value(((const uint8_t *)kv)[rows[i] * C + c]) *
                                             (double)kv_scales[rows[i]]
                                       : bf16_value(((const uint16_t *)kv)[rows[i] * C + c]);
                    dot += bf16_value(qh[c]) * vc;
                }
                logit[i] = sm * dot;
                if (logit[i] > mx) mx = logit[i];
            }
            for (long i = 0; i < n; ++i) den += exp(logit[i] - mx);
            for (long c = 0; c < C; ++c) v[c] = 0.0;
            for (long i = 0; i < n; ++i) {
                double pw = exp(logit[i] - mx) / den;
                for (long c = 0; c < C; ++c) {
                    double vc = kv_fp8 ? e4m3_value(((const uint8_t *)kv)[rows[i] * C + c]) *
                                             (double)kv_scales[rows[i]]
                                       : bf16_value(((const uint16_t *)kv)[rows[i] * C + c]);
                    v[c] += pw * vc;
                }
            }
            for (long c = 0; c < C; ++c) oh[c] = n ? (float)v[c] : 0.0f;
            if (lse) lse[r * H + h] = n ? (float)(mx + log(den)) : -INFINITY;
        }
        free(rows);
        free(logit);
        free(v);
    }
}

/* ---------------------------------------------------------------- dense masked cross-check */

/* mod.rs, Glm5NextDsaKernels::topk_to_mask and MASKED_ATTN_MAX_KEYS (the selection turned into
 * a token mask that a dense masked attention takes, as a second check of the sparse decode).
 * Reading: mask[r, t] = 1 when some slot of token_ids[r] holds t (0 <= t < S), else 0.
 * Layouts: token_ids [Q, W] i32; mask [Q, S] u8. */
void orc_topk_to_mask(int Q, int W, int S, const int32_t *token_ids, uint8_t *mask) {
    for (long r = 0; r < Q; ++r) {
        for (long t = 0; t < S; ++t) mask[r * S + t] = 0;
        for (long i = 0; i < W; ++i) {
            long t = token_ids[r * W + i];
            if (t >= 0 && t < S) mask[r * S + t] = 1;
        }
    }
}

/* mod.rs, mla_masked_attn: attention of row r, head h over every token t < S of sequence
 * b = row_seq[r] with mask[r, t] = 1, the whole [S] score row at once: logit_t =
 * sm * q_abs[r,h,:] . v_t, out = sum_t softmax(logit)_t v_t, lse = log sum exp(logit), with
 * latent rows addressed as orc_sparse_mla addresses them (a token whose row is absent from
 * the table is skipped). A row with no token: out = 0, lse = -inf.
 * Layouts: q_abs [Q,H,C] bf16; mask [Q,S] u8; kv [rows, C] bf16 or e4m3 (+ kv_scales [rows]);
 * out [Q,H,C] f32; lse [Q,H] f32. */
void orc_masked_attn(int Q, int H, int C, int S, double sm, const uint16_t *q_abs,
                     const uint8_t *mask, const int32_t *row_seq, const void *kv, int kv_fp8,
                     const float *kv_scales, const int32_t *block_table, int max_blocks,
                     int block_size, float *out, float *lse) {
    long r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < Q; ++r) {
        long b = row_seq[r];
        double *logit = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        long *rows = (long *)malloc(sizeof(long) * (size_t)(S > 0 ? S : 1));
        double *v = (double *)malloc(sizeof(double) * (size_t)C);
        for (long t = 0; t < S; ++t) {
            rows[t] = -1;
            if (!mask[r * S + t]) continue;
            if (block_table) {
                long blk = t / block_size;
                if (blk < max_blocks && block_table[b * max_blocks + blk] >= 0)
                    rows[t] = (long)block_table[b * max_blocks + blk] * block_size + t % block_size;
            } else {
                rows[t] = b * (long)S + t;
            }
        }
        for (long h = 0; h < H; ++h) {
            const uint16_t *qh = q_abs + (r * H + h) * C;
            double mx = -INFINITY, den = 0.0;
            long n = 0;
            for (long t = 0; t < S; ++t) {
                if (rows[t] < 0) continue;
                double dot = 0.0;
                for (long c = 0; c < C; ++c) {
                    double vc = kv_fp8 ? e4m3_value(((const uint8_t *)kv)[rows[t] * C + c]) *
                                             (double)kv_scales[rows[t]]
                                       : bf16_value(((const uint16_t *)kv)[rows[t] * C + c]);
                    dot += bf16_value(qh[c]) * vc;
                }
                logit[t] = sm * dot;
                if (logit[t] > mx) mx = logit[t];
                ++n;
            }
            for (long t = 0; t < S; ++t)
                if (rows[t] >= 0) den += exp(logit[t] - mx);
            for (long c = 0; c < C; ++c) v[c] = 0.0;
            for (long t = 0; t < S; ++t) {
                if (rows[t] < 0) continue;
                double pw = exp(logit[t] - mx) / den;
                for (long c = 0; c < C; ++c) {
                    double vc = kv_fp8 ? e4m3_value(((const uint8_t *)kv)[rows[t] * C + c]) *
                                             (double)kv_scales[rows[t]]
                                       : bf16_value(((const uint16_t *)kv)[rows[t] * C + c]);
                    v[c] += pw * vc;
                }
            }
            for (long c = 0; c < C; ++c) out[(r * H + h) * C + c] = n ? (float)v[c] : 0.0f;
            if (lse) lse[r * H + h] = n ? (float)(mx + log(den)) : -INFINITY;
        }
        free(logit);
        free(rows);
        free(v);
    }
}

/* ---------------------------------------------------------------- decode-time cache maintenance */

/* mod.rs, Glm5NextDsaKernels::k_norm: indexer.k_norm is a LayerNorm with a bias (not an
 * RMSNorm), applied in place to bf16 rows with bf16 weight and bias.
 * Reading: per row the mean and the biased variance over the D values;
 * y = (x - mean) / sqrt(var + eps) * weight + bias, in double, rounded once to bf16.
 * Layouts: x [rows, D] bf16 (in place); weight, bias [D] bf16. */
void orc_layer_norm(long rows, int D, uint16_t *x, const uint16_t *weight, const uint16_t *bias,
                    double eps) {
    for (long r = 0; r < rows; ++r) {
        uint16_t *row = x + r * D;
        double mean = 0.0, var = 0.0;
        for (int d = 0; d < D; ++d) mean += bf16_value(row[d]);
        mean /= D;
        for (int d = 0; d < D; ++d) var += (bf16_value(row[d]) - mean) * (bf16_value(row[d]) - mean);
        var /= D;
        double inv = 1.0 / sqrt(var + eps);
        for (int d = 0; d < D; ++d)
            row[d] = bf16_from_float(
                (float)((bf16_value(row[d]) - mean) * inv * bf16_value(weight[d]) + bf16_value(bias[d])));
    }
}

/* mod.rs, Glm5NextDsaKernels::indexer_store: the staged indexer row is copied to a device-side
 * position and marked valid.
 * Reading: the staged row of sequence b is its new token's key and gate; for
 * 0 <= pos[b] < S: k_cache[b,pos] = k_row[b], gate_cache[b,pos] = gate_row[b],
 * valid[b,pos] = 1; any other pos stores nothing.
 * Layouts: pos [B] i32; k_row, gate_row [B, D] bf16; k_cache, gate_cache [B, S, D] bf16;
 * valid [B, S] u8. */
void orc_indexer_store(int B, int S, int D, const int32_t *pos, const uint16_t *k_row,
                       const uint16_t *gate_row, uint16_t *k_cache, uint16_t *gate_cache,
                       uint8_t *valid) {
    for (long b = 0; b < B; ++b) {
        long t = pos[b];
        if (t < 0 || t >= S) continue;
        for (int d = 0; d < D; ++d) {
            k_cache[(b * S + t) * D + d] = k_row[b * D + d];
            gate_cache[(b * S + t) * D + d] = gate_row[b * D + d];
        }
        valid[b * S + t] = 1;
    }
}

/* mod.rs, Glm5NextDsaKernels::write_geom: the selector geometry derived on the device from
 * seq_len, so a captured graph replays over the live context.
 * Reading (decode, one query row per sequence): row_seq[b] = b, row_pos[b] = seq_len[b] - 1. */
void orc_write_geom(int B, const int32_t *seq_len, int32_t *row_seq, int32_t *row_pos) {
    for (int b = 0; b < B; ++b) {
        row_seq[b] = b;
        row_pos[b] = seq_len[b] - 1;
    }
}

/* The pool that a newly stored token completes, kept up to date at decode time (mod.rs
 * "Checkpoint and kernel facts": pooling starts at first_key and a pool counts only when
 * all its slots are valid; "Shape of the pipeline": pool keys, indices and validity).
 * Reading: token pos of sequence b completes pool p = (pos - first_key + 1)/KP - 1 when
 * pos >= first_key, (pos - first_key + 1) % KP == 0 and p < P. That pool's key and validity
 * are computed exactly as kpool_compress computes them, and a valid pool is appended to the
 * compacted id list (ids[b, n_valid[b]] = p, n_valid[b] += 1) unless the list already ends at
 * p or beyond; any other position changes nothing.
 * Layouts as orc_kpool_compress and orc_compact_pools; pos [B] i32. */
void orc_pool_append(int B, int S, int D, int KP, int first_key, const int32_t *pos,
                     const uint16_t *k, const uint16_t *gate, const float *ape,
                     const uint8_t *valid, uint16_t *pool_keys, uint8_t *pool_valid,
                     int32_t *ids, int32_t *n_valid) {
    long P = orc_num_pools(S, first_key, KP);
    for (long b = 0; b < B; ++b) {
        long t = pos[b];
        if (t < first_key || t >= S || (t - first_key + 1) % KP != 0) continue;
        long p = (t - first_key + 1) / KP - 1;
        if (p >= P) continue;
        compress_pool(b, p, P, S, D, KP, first_key, k, gate, ape, valid, pool_keys, pool_valid);
        long n = n_valid[b];
        if (pool_valid[b * P + p] && (n == 0 || ids[b * P + n - 1] < p) && n < P) {
            ids[b * P + n] = (int32_t)p;
            n_valid[b] = (int32_t)(n + 1);
        }
    }
}

/* ---------------------------------------------------------------- host weight transforms */

static void put_msg(char *msg, int msg_len, const char *text) {
    if (msg && msg_len > 0) {
        strncpy(msg, text, (size_t)msg_len - 1);
        msg[msg_len - 1] = 0;
    }
}

/* One element of either absorption (build.rs, "The transforms" 1 and 3): the binary32 sum,
 * started at 0 and taken over r = 0, 1, ..., n-1 in that order, of the rounded products
 * a[r*sa] * b[r*sb]. The bit-exact absorption fixes exactly this arithmetic (the file is
 * compiled with -ffp-contract=off, so no product is fused into its addition). */
static float dot_f32_ascending(const float *a, long sa, const float *b, long sb, long n) {
    float sum = 0.0f;
    for (long r = 0; r < n; ++r) {
        float term = a[r * sa] * b[r * sb];
        sum = sum + term;
    }
    return sum;
}

/* build.rs, absorb_q: q_absorb[h*kvl + c][k] = sum over r < nope of
 * kv_b[h*(nope+vd) + r][c] * q_b[h*nope + r][k], each element by dot_f32_ascending. Refuses
 * wrong element counts (q_b must be [heads*(nope+rope), ql], kv_b [heads*(nope+vd), kvl]) and
 * a nonzero rope width. Returns 0, or 1 (q_b count), 2 (kv_b count), 3 (rope). out is
 * [heads*kvl, ql]. */
int orc_absorb_q(int heads, int nope, int rope, int vd, int kvl, int ql, const float *q_b,
                 long q_b_len, const float *kv_b, long kv_b_len, float *out, char *msg,
                 int msg_len) {
    if (q_b_len != (long)heads * (nope + rope) * ql) {
        put_msg(msg, msg_len, "q_b element count does not match heads*qk_head_dim*q_lora_rank");
        return 1;
    }
    if (kv_b_len != (long)heads * (nope + vd) * kvl) {
        put_msg(msg, msg_len, "kv_b element count does not match heads*(nope+v)*kv_lora_rank");
        return 2;
    }
    if (rope != 0) {
        put_msg(msg, msg_len, "absorption is defined for NoPE only (rope width must be 0)");
        return 3;
    }
    for (long h = 0; h < heads; ++h)
        for (long c = 0; c < kvl; ++c)
            for (long k = 0; k < ql; ++k)
                out[(h * kvl + c) * ql + k] =
                    dot_f32_ascending(kv_b + (h * (nope + vd)) * kvl + c, kvl,   /* over r: kv_b[.][c] */
                                      q_b + (h * nope) * ql + k, ql,             /* over r: q_b[.][k] */
                                      nope);
    return 0;
}

/* build.rs, absorb_o: o_absorb[i][h*kvl + c] = sum over r < vd of
 * o_proj[i][h*vd + r] * kv_b[h*(nope+vd) + nope + r][c], each element by dot_f32_ascending.
 * Refuses a nonzero rope width and wrong counts (o_local [hidden, heads*vd], kv_b_local
 * [heads*(nope+vd), kvl]). Returns 0, or 3 (rope), 1 (o_proj count), 2 (kv_b count), checked
 * in that order. out is [hidden, heads*kvl]. */
int orc_absorb_o(int heads, int nope, int rope, int vd, int kvl, int hidden, const float *o_local,
                 long o_len, const float *kv_b_local, long kv_len, float *out, char *msg,
                 int msg_len) {
    if (rope != 0) {
        put_msg(msg, msg_len, "absorption is defined for NoPE only (rope width must be 0)");
        return 3;
    }
    long in_w = (long)heads * vd, out_w = (long)heads * kvl;
    if (o_len != (long)hidden * in_w) {
        put_msg(msg, msg_len, "o_proj element count does not match hidden*heads*v_head_dim");
        return 1;
    }
    if (kv_len != (long)heads * (nope + vd) * kvl) {
        put_msg(msg, msg_len, "kv_b element count does not match heads*(nope+v)*kv_lora_rank");
        return 2;
    }
    for (long i = 0; i < hidden; ++i)
        for (long h = 0; h < heads; ++h)
            for (long c = 0; c < kvl; ++c)
                out[i * out_w + h * kvl + c] =
                    dot_f32_ascending(o_local + i * in_w + h * vd, 1,                   /* o_proj[i][h*vd + r] */
                                      kv_b_local + (h * (nope + vd) + nope) * kvl + c, kvl,  /* kv_b[.][c] */
                                      vd);
    return 0;
}

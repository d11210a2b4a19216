// absorb.cpp -- host-side load-time weight transforms (build.rs, absorb_q, absorb_o, up_bf16).
//
// Compiled with -ffp-contract=off: each output element is accumulated in f32 as
// acc = acc + (a * b), r ascending, inside one thread, so the result is bit-identical for
// any thread count (build.rs, absorb_q_rows: the absorb_q_bit_exact property).
#include <cerrno>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "dsa.h"
#include "dsa_host.hpp"

namespace dsa_host {

// Worker threads: an explicit positive count, else the DSA_ABSORB_THREADS environment variable
// when it parses as a positive integer, else the hardware concurrency; clamped to 1..rows
// (build.rs, absorb_threads).
size_t absorb_threads(int requested, size_t rows) {
    size_t want = 0;
    if (requested > 0) {
        want = (size_t)requested;
    } else {
        const char *env = std::getenv("DSA_ABSORB_THREADS");
        if (env) {
            while (*env == ' ' || *env == '\t' || *env == '\n') ++env;
            char *end = nullptr;
            errno = 0;
            const long long v = std::strtoll(env, &end, 10);
            while (end && (*end == ' ' || *end == '\t' || *end == '\n')) ++end;
            if (errno == 0 && end && *end == 0 && end != env && v > 0) want = (size_t)v;
        }
        if (want == 0) {
            const unsigned hc = std::thread::hardware_concurrency();
            want = hc > 0 ? hc : 1;
        }
    }
    if (rows == 0) rows = 1;
    if (want < 1) want = 1;
    if (want > rows) want = rows;
    return want;
}

template <class F>
void run_spans(size_t rows, size_t threads, F &&body) {
    if (threads <= 1) {
        body(0, rows);
        return;
    }
    const size_t per = (rows + threads - 1) / threads;
    std::vector<std::thread> pool;
    for (size_t r0 = 0; r0 < rows; r0 += per) {
        const size_t r1 = r0 + per < rows ? r0 + per : rows;
        pool.emplace_back([&body, r0, r1] { body(r0, r1); });
    }
    for (auto &t : pool) t.join();
}

}  // namespace dsa_host

extern "C" {

int dsa_absorb_q(const dsa_config *cfg, const float *q_b, size_t q_b_len, const float *kv_b,
                 size_t kv_b_len, int full_heads, int threads, float *out, size_t out_len) {
    using dsa_host::set_error;
    dsa_host::clear_error();
    if (!cfg) return set_error(DSA_ERR_NULL_ARG, "config is NULL");
    if (full_heads < 0 || cfg->qk_nope_head_dim < 0 || cfg->qk_rope_head_dim < 0 ||
        cfg->v_head_dim < 0 || cfg->kv_lora_rank < 0 || cfg->q_lora_rank < 0)
        return set_error(DSA_ERR_BAD_SIZE, "absorb_q: negative dimension");
    const size_t nope = cfg->qk_nope_head_dim, vd = cfg->v_head_dim, kvl = cfg->kv_lora_rank,
                 ql = cfg->q_lora_rank, rope = cfg->qk_rope_head_dim, heads = full_heads;
    if (q_b_len != heads * (nope + rope) * ql)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_q: q_b has %zu elements, the config needs %zu",
                         q_b_len, heads * (nope + rope) * ql);
    if (kv_b_len != heads * (nope + vd) * kvl)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_q: kv_b has %zu elements, the config needs %zu",
                         kv_b_len, heads * (nope + vd) * kvl);
    if (rope != 0)
        return set_error(DSA_ERR_ROPE_UNSUPPORTED,
                         "absorb_q: only NoPE can be absorbed (qk_rope_head_dim is %zu)", rope);
    const size_t rows = heads * kvl;
    if (out_len != rows * ql)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_q: out has %zu elements, needs %zu", out_len,
                         rows * ql);
    if (rows * ql == 0) return DSA_OK;
    if (!q_b || !kv_b || !out) return set_error(DSA_ERR_NULL_ARG, "absorb_q: a buffer is NULL");
    const size_t nt = dsa_host::absorb_threads(threads, rows);
    dsa_host::run_spans(rows, nt, [&](size_t r0, size_t r1) {
        for (size_t row = r0; row < r1; ++row) {
            const size_t h = row / kvl, c = row % kvl;
            float *acc = out + row * ql;
            for (size_t k = 0; k < ql; ++k) acc[k] = 0.0f;
            for (size_t r = 0; r < nope; ++r) {
                const float wv = kv_b[(h * (nope + vd) + r) * kvl + c];
                const float *qrow = q_b + (h * nope + r) * ql;
                for (size_t k = 0; k < ql; ++k) acc[k] = acc[k] + qrow[k] * wv;
            }
        }
    });
    return DSA_OK;
}

int dsa_absorb_o(const dsa_config *cfg, const float *o_local, size_t o_len,
                 const float *kv_b_local, size_t kv_len, int local_heads, int threads,
                 float *out, size_t out_len) {
    using dsa_host::set_error;
    dsa_host::clear_error();
    if (!cfg) return set_error(DSA_ERR_NULL_ARG, "config is NULL");
    if (local_heads < 0 || cfg->qk_nope_head_dim < 0 || cfg->v_head_dim < 0 ||
        cfg->kv_lora_rank < 0 || cfg->hidden < 0 || cfg->qk_rope_head_dim < 0)
        return set_error(DSA_ERR_BAD_SIZE, "absorb_o: negative dimension");
    if (cfg->qk_rope_head_dim != 0)
        return set_error(DSA_ERR_ROPE_UNSUPPORTED,
                         "absorb_o: only NoPE can be absorbed (qk_rope_head_dim is %d)",
                         cfg->qk_rope_head_dim);
    const size_t nope = cfg->qk_nope_head_dim, vd = cfg->v_head_dim, kvl = cfg->kv_lora_rank,
                 hidden = cfg->hidden, heads = local_heads;
    const size_t in_w = heads * vd, out_w = heads * kvl;
    if (o_len != hidden * in_w)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_o: o_proj has %zu elements, expected %zu",
                         o_len, hidden * in_w);
    if (kv_len != heads * (nope + vd) * kvl)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_o: kv_b slice has %zu elements, expected %zu",
                         kv_len, heads * (nope + vd) * kvl);
    if (out_len != hidden * out_w)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_o: out has %zu elements, needs %zu", out_len,
                         hidden * out_w);
    if (hidden * out_w == 0) return DSA_OK;
    if (!o_local || !kv_b_local || !out) return set_error(DSA_ERR_NULL_ARG, "absorb_o: a buffer is NULL");
    const size_t nt = dsa_host::absorb_threads(threads, hidden);
    dsa_host::run_spans(hidden, nt, [&](size_t i0, size_t i1) {
        for (size_t i = i0; i < i1; ++i) {
            float *dst_row = out + i * out_w;
            const float *src_row = o_local + i * in_w;
            for (size_t k = 0; k < out_w; ++k) dst_row[k] = 0.0f;
            for (size_t h = 0; h < heads; ++h) {
                float *dst = dst_row + h * kvl;
                const size_t v_base = h * (nope + vd) + nope;
                for (size_t r = 0; r < vd; ++r) {
                    const float wv = src_row[h * vd + r];
                    const float *src = kv_b_local + (v_base + r) * kvl;
                    for (size_t c = 0; c < kvl; ++c) dst[c] = dst[c] + wv * src[c];
                }
            }
        }
    });
    return DSA_OK;
}

void dsa_f32_to_bf16_rne(const float *src, uint16_t *dst, size_t n) {
    if (!src || !dst) return;
    for (size_t i = 0; i < n; ++i) {
        uint32_t u;
        std::memcpy(&u, &src[i], sizeof u);
        if ((u & 0x7fffffffu) > 0x7f800000u) {
            dst[i] = (uint16_t)((u >> 16) | 0x40u);
            continue;
        }
        const uint32_t lsb = (u >> 16) & 1u;
        dst[i] = (uint16_t)((u + 0x7fffu + lsb) >> 16);
    }
}

}  // extern "C"

// absorb.cpp -- host-side load-time weight transforms (build.rs, "The transforms" 1 and 3,
// absorb_q, absorb_o) and the bf16 upload rounding (up_bf16).
//
// Both transforms are products over the no-position (or value) width r of one head:
//   q_absorb[h*kvl + c][k]   = sum_{r < nope} kv_b[h*(nope+vd) + r][c] * q_b[h*nope + r][k]
//   o_absorb[i][h*kvl + c]   = sum_{r < vd}   o_proj[i][h*vd + r] * kv_b[h*(nope+vd) + nope + r][c]
// The pages require the result to be bit-identical for any number of threads, which fixes the
// arithmetic of each element: a binary32 sum from 0 over r ascending, each product rounded
// before it is added (this file is compiled with -ffp-contract=off). Everything else is free:
// here the work is cut into tiles (one head times a block of output columns), each tile owned
// by one thread and swept r-outermost, so a tile's accumulators stay in cache while the
// weight rows stream past once.
#include <algorithm>
#include <cctype>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "dsa.h"
#include "dsa_host.hpp"

namespace {

constexpr size_t kColBlock = 64;   // output columns per tile (absorb_q: k; absorb_o: rows i)

// A positive integer from the environment (surrounding blanks allowed), else 0.
long long env_positive(const char *name) {
    const char *raw = std::getenv(name);
    if (raw == nullptr) return 0;
    std::string t(raw);
    const auto blank = [](unsigned char ch) { return std::isspace(ch) != 0; };
    while (!t.empty() && blank(t.back())) t.pop_back();
    size_t i = 0;
    while (i < t.size() && blank(t[i])) ++i;
    t.erase(0, i);
    if (t.empty() || t.size() > 18) return 0;
    for (unsigned char ch : t)
        if (ch < '0' || ch > '9') return 0;
    return std::atoll(t.c_str());
}

// Worker count (build.rs, absorb_threads): the explicit argument when positive, else
// DSA_ABSORB_THREADS when it holds a positive integer, else the hardware concurrency; never
// more workers than work items, never fewer than one. It changes speed only, not results.
size_t worker_count(int requested, size_t items) {
    long long n = requested > 0 ? requested : env_positive("DSA_ABSORB_THREADS");
    if (n <= 0) n = (long long)std::thread::hardware_concurrency();
    const long long cap = (long long)std::max<size_t>(items, 1);
    return (size_t)std::clamp<long long>(n, 1, cap);
}

// Run body(item) for item in [0, items) on `workers` threads, items dealt round-robin.
template <class F>
void parallel_items(size_t items, size_t workers, F &&body) {
    if (workers <= 1) {
        for (size_t it = 0; it < items; ++it) body(it);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(workers);
    for (size_t w = 0; w < workers; ++w)
        pool.emplace_back([&body, w, workers, items] {
            for (size_t it = w; it < items; it += workers) body(it);
        });
    for (auto &t : pool) t.join();
}

}  // namespace

extern "C" {

int dsa_absorb_q(const dsa_config *cfg, const float *q_b, size_t q_b_len, const float *kv_b,
                 size_t kv_b_len, int full_heads, int threads, float *out, size_t out_len) {
    using dsa_host::set_error;
    dsa_host::clear_error();
    if (!cfg) return set_error(DSA_ERR_NULL_ARG, "config is NULL");
    if (full_heads < 0 || cfg->qk_nope_head_dim < 0 || cfg->qk_rope_head_dim < 0 ||
        cfg->v_head_dim < 0 || cfg->kv_lora_rank < 0 || cfg->q_lora_rank < 0)
        return set_error(DSA_ERR_BAD_SIZE, "absorb_q: negative dimension");
    const size_t heads = (size_t)full_heads, nope = (size_t)cfg->qk_nope_head_dim,
                 rope = (size_t)cfg->qk_rope_head_dim, vd = (size_t)cfg->v_head_dim,
                 kvl = (size_t)cfg->kv_lora_rank, ql = (size_t)cfg->q_lora_rank;
    if (q_b_len != heads * (nope + rope) * ql)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_q: q_b has %zu elements, the config needs %zu",
                         q_b_len, heads * (nope + rope) * ql);
    if (kv_b_len != heads * (nope + vd) * kvl)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_q: kv_b has %zu elements, the config needs %zu",
                         kv_b_len, heads * (nope + vd) * kvl);
    if (rope != 0)
        return set_error(DSA_ERR_ROPE_UNSUPPORTED,
                         "absorb_q: only NoPE can be absorbed (qk_rope_head_dim is %zu)", rope);
    if (out_len != heads * kvl * ql)
        return set_error(DSA_ERR_ELEM_COUNT, "absorb_q: out has %zu elements, needs %zu", out_len,
                         heads * kvl * ql);
    if (out_len == 0) return DSA_OK;
    if (!q_b || !kv_b || !out) return set_error(DSA_ERR_NULL_ARG, "absorb_q: a buffer is NULL");
    // Tile (h, kb): output rows h*kvl .. h*kvl + kvl - 1, columns kb*kColBlock .. + kColBlock.
    const size_t kblocks = (ql + kColBlock - 1) / kColBlock;
    const size_t tiles = heads * kblocks;
    parallel_items(tiles, worker_count(threads, tiles), [&](size_t tile) {
        const size_t h = tile / kblocks, k0 = (tile % kblocks) * kColBlock;
        const size_t kn = std::min(kColBlock, ql - k0);
        float *const t0 = out + h * kvl * ql + k0;
        for (size_t c = 0; c < kvl; ++c) std::memset(t0 + c * ql, 0, kn * sizeof(float));
        for (size_t r = 0; r < nope; ++r) {
            const float *const weights = kv_b + (h * (nope + vd) + r) * kvl;   // kv_b row, over c
            const float *const qv = q_b + (h * nope + r) * ql + k0;           // q_b row, over k
            for (size_t c = 0; c < kvl; ++c) {
                const float wc = weights[c];
                float *const o = t0 + c * ql;
                for (size_t j = 0; j < kn; ++j) o[j] = o[j] + wc * qv[j];
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
    const size_t heads = (size_t)local_heads, nope = (size_t)cfg->qk_nope_head_dim,
                 vd = (size_t)cfg->v_head_dim, kvl = (size_t)cfg->kv_lora_rank,
                 hidden = (size_t)cfg->hidden;
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
    if (out_len == 0) return DSA_OK;
    if (!o_local || !kv_b_local || !out)
        return set_error(DSA_ERR_NULL_ARG, "absorb_o: a buffer is NULL");
    // Tile (h, ib): output rows ib*kColBlock .. + kColBlock, columns h*kvl .. h*kvl + kvl - 1.
    const size_t iblocks = (hidden + kColBlock - 1) / kColBlock;
    const size_t tiles = heads * iblocks;
    parallel_items(tiles, worker_count(threads, tiles), [&](size_t tile) {
        const size_t h = tile / iblocks, i0 = (tile % iblocks) * kColBlock;
        const size_t in_ = std::min(kColBlock, hidden - i0);
        for (size_t i = i0; i < i0 + in_; ++i) std::memset(out + i * out_w + h * kvl, 0, kvl * sizeof(float));
        for (size_t r = 0; r < vd; ++r) {
            const float *const vrow = kv_b_local + (h * (nope + vd) + nope + r) * kvl;  // over c
            for (size_t i = i0; i < i0 + in_; ++i) {
                const float oi = o_local[i * in_w + h * vd + r];
                float *const o = out + i * out_w + h * kvl;
                for (size_t c = 0; c < kvl; ++c) o[c] = o[c] + oi * vrow[c];
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

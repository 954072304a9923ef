// Host-only part of libmsa: argument validation, workspace layout, status
// strings. Holds no HIP calls, so every error path can be exercised on a
// machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "msa_internal.h"

namespace msa {

static thread_local char g_err[512] = "";

msa_status fail(msa_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_err[0] = '\0'; }

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

msa_status check_config(const msa_config *c) {
    if (!c) return fail(MSA_ERR_INVALID_ARG, "cfg is NULL");
    if (c->num_kv_groups < 1) return fail(MSA_ERR_INVALID_ARG, "num_kv_groups must be >= 1");
    if (c->heads_per_group < 1) return fail(MSA_ERR_INVALID_ARG, "heads_per_group must be >= 1");
    if (c->head_dim < 1 || c->index_dim < 1 || c->block_size < 1 || c->topk < 1)
        return fail(MSA_ERR_INVALID_ARG, "head_dim, index_dim, block_size and topk must be >= 1");
    if (!(c->softmax_scale >= 0.0f) || isinf(c->softmax_scale))
        return fail(MSA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    if (c->index_dtype != MSA_BF16 && c->index_dtype != MSA_FP8_E4M3)
        return fail(MSA_ERR_INVALID_ARG, "index_dtype %d is not a msa_dtype", c->index_dtype);
    if (c->head_dim != kHeadDim)
        return fail(MSA_ERR_UNSUPPORTED, "head_dim %d unsupported (need 128)", c->head_dim);
    if (c->index_dim != kIndexDim)
        return fail(MSA_ERR_UNSUPPORTED, "index_dim %d unsupported (need 128)", c->index_dim);
    if (c->block_size != kBlock)
        return fail(MSA_ERR_UNSUPPORTED, "block_size %d unsupported (need 128)", c->block_size);
    if (c->topk > kMaxTopk)
        return fail(MSA_ERR_UNSUPPORTED, "topk %d unsupported (need 1..64)", c->topk);
    if (c->heads_per_group > kMaxHeadsPerGroup)
        return fail(MSA_ERR_UNSUPPORTED, "heads_per_group %d unsupported (need 1..16)",
                    c->heads_per_group);
    if ((int64_t)c->num_kv_groups * c->heads_per_group > 4096)
        return fail(MSA_ERR_UNSUPPORTED, "more than 4096 query heads");
    return MSA_OK;
}

static msa_status check_dims(int32_t B, int32_t T, int32_t Nmax) {
    if (B < 0 || T < 0) return fail(MSA_ERR_INVALID_ARG, "B and T must be >= 0");
    if (B > 65535) return fail(MSA_ERR_UNSUPPORTED, "B = %d exceeds 65535", B);
    if (B > 0 && T > 0 && Nmax < 1) return fail(MSA_ERR_INVALID_ARG, "Nmax must be >= 1");
    if (Nmax < 0) return fail(MSA_ERR_INVALID_ARG, "Nmax must be >= 0");
    return MSA_OK;
}

bool index_uses_pooled(const msa_config *cfg, int32_t B, int32_t T) {
    const int64_t rows = (int64_t)T * cfg->num_kv_groups;
    if (rows <= kScanMaxRows || cfg->topk > kPrefillRegTopk) return true;
    return (rows + kIdxTileRows - 1) / kIdxTileRows * B < kIdxRegMinWgs;
}

IndexWs index_ws(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax) {
    IndexWs w{};
    w.nb_max = ((int64_t)Nmax + kBlock - 1) / kBlock;
    w.pooled_off = 0;
    const bool pooled = index_uses_pooled(cfg, B, T);
    w.pooled_bytes =
        pooled ? (size_t)B * (size_t)T * (size_t)cfg->num_kv_groups * (size_t)w.nb_max * 4 : 0;
    w.total = round_up(w.pooled_bytes, kWsAlign);
    return w;
}

int32_t prefill_entries_per_tile(int32_t R) {
    return kPfRounds * kPfWaves * kPfNq * (16 / R);
}

PrefillWs prefill_ws(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax, bool backward) {
    PrefillWs w{};
    const int64_t G = cfg->num_kv_groups, K = cfg->topk, R = cfg->heads_per_group;
    w.kv_major = backward || (int64_t)B * T * G >= kPfKvMajorMinRows;
    if (!w.kv_major || B == 0 || T == 0) return w;
    // One pass covers every group and `rows` query rows of every sequence: the
    // largest power of two of rows (or all T) whose partials fit
    // kPfPartialBudget, with at most 2^24 (sequence, row, group) units. (Passes
    // of one group whose queries stay in the last-level cache were measured
    // slower: the list build is paid per pass.)
    // Per (row, group, slot, head): the forward keeps O / l in bf16 and (m, l);
    // the backward keeps a dq partial in bf16.
    // (The backward's per-tile dk/dv partials, 2*S*d fp32 per tile of
    // entries_per_tile entries, add 2*S*d*4 / entries_per_tile bytes per slot.)
    const size_t part_row =
        (size_t)B * G * K *
        (backward ? (size_t)R * kHeadDim * 2 +
                        (size_t)2 * kBlock * kHeadDim * 4 / prefill_entries_per_tile(R)
                  : (size_t)R * (kHeadDim * 2 + 8));
    // The list build keeps a row bitmap and its word prefixes per list: 8
    // bytes per 32 rows of each of the B*G*nb lists, within kPfBitmapBudget.
    const int64_t nb = ((int64_t)Nmax + kBlock - 1) / kBlock;
    const size_t bits_row = (size_t)B * G * nb / 4 + 1;
    const int64_t max_units = (int64_t)1 << 24;
    int64_t rows = 1;
    auto fits = [&](int64_t r) {
        return (size_t)r * part_row <= kPfPartialBudget && (size_t)r * bits_row <= kPfBitmapBudget &&
               r * B * G <= max_units;
    };
    while (rows * 2 <= T && fits(rows * 2)) rows *= 2;
    if (fits(T)) rows = T;
    const int64_t groups = G;
    w.rows = (int32_t)rows;
    w.groups = (int32_t)groups;
    w.entries_per_tile = prefill_entries_per_tile(cfg->heads_per_group);
    w.nb_max = ((int64_t)Nmax + kBlock - 1) / kBlock;
    w.nlists = (int64_t)B * groups * w.nb_max;
    w.nslots = (int64_t)B * rows * groups * K;
    if (!backward) {
        // A short prefill has few entries: fewer rounds per tile (down to one
        // per wave), so that a pass still has about kPfFillTiles tiles to
        // spread over the chip. (The backward keeps full tiles: its per-tile
        // dk/dv partials are budgeted for them.)
        const int32_t round = kPfWaves * kPfNq * (16 / (int32_t)R);
        while (w.entries_per_tile > round && w.nslots / w.entries_per_tile < kPfFillTiles)
            w.entries_per_tile /= 2;
    }
    w.max_tiles = (w.nslots + w.entries_per_tile - 1) / w.entries_per_tile + w.nlists;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = round_up(off + bytes, kWsAlign); return o; };
    w.bit_words = (int32_t)((rows + 31) / 32);
    w.bits_off = take((size_t)w.nlists * w.bit_words * 4);
    w.wpre_off = take((size_t)w.nlists * w.bit_words * 4);
    w.counts_off = take((size_t)w.nlists * 4);
    w.offsets_off = take((size_t)(w.nlists + 1) * 4);
    w.tile_first_off = take((size_t)(w.nlists + 1) * 4);
    w.tile_map_off = take((size_t)w.max_tiles * 4);
    w.list_off = take((size_t)w.nslots * 4);
    if (backward) {
        w.part_o_off = take((size_t)w.nslots * R * kHeadDim * 2);  // dq partials, bf16
        w.part_ml_off = take((size_t)w.max_tiles * 2 * kBlock * kHeadDim * 4);  // dk/dv per tile
        w.delta_off = take((size_t)B * T * G * R * 4);            // dout . out per (row, head)
    } else {
        w.part_o_off = take((size_t)w.nslots * R * kHeadDim * 2);
        w.part_ml_off = take((size_t)w.nslots * R * 8);
    }
    w.trash_off = take(kPfTrashBytes);
    w.total = off;
    return w;
}

int32_t decode_waves(const msa_config *cfg, int32_t B) {
    const int64_t splits16 = (4 * cfg->topk + 15) / 16;
    return (int64_t)B * cfg->num_kv_groups * splits16 >= kDecodeFillWorkgroups ? 16 : 8;
}

int32_t decode_splits(const msa_config *cfg, int32_t B) {
    const int32_t w = decode_waves(cfg, B);
    return (4 * cfg->topk + w - 1) / w;
}

DecodeWs decode_ws(const msa_config *cfg, int32_t B, int32_t Nmax, bool with_index) {
    DecodeWs w{};
    w.nb_max = ((int64_t)Nmax + kBlock - 1) / kBlock;
    w.pooled_off = 0;
    // Pooled block scores of every (sequence, group) row, whichever index
    // kernel writes them (the streaming one for G <= kScanMaxRows, the MFMA
    // prefill one above).
    const size_t pooled =
        with_index ? round_up((size_t)B * cfg->num_kv_groups * (size_t)w.nb_max * 4, kWsAlign) : 0;
    const size_t units =
        (size_t)B * cfg->num_kv_groups * decode_splits(cfg, B) * cfg->heads_per_group;
    w.part_o_off = pooled;
    // (m, l) directly after O (units * 512 bytes keep the alignment): the
    // decode kernels treat the partials as one run of units * (d + 2) words.
    w.part_ml_off = w.part_o_off + units * kHeadDim * 4;
    w.counters_off = round_up(w.part_ml_off + units * 2 * 4, kWsAlign);
    const size_t counters = with_index ? (size_t)B * cfg->num_kv_groups * 4 : 0;
    w.total = round_up(w.counters_off + counters, kWsAlign);
    return w;
}

static msa_status check_ws(const void *ws, size_t have, size_t need) {
    if (need == 0) return MSA_OK;
    if (!ws) return fail(MSA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if (!aligned(ws, kWsAlign)) return fail(MSA_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (have < need)
        return fail(MSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    return MSA_OK;
}

msa_status check_index_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                            const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                            const int32_t *q_start, const int32_t *sel, const float *sel_scores,
                            const void *workspace, size_t ws_bytes) {
    msa_status s = check_config(cfg);
    if (s != MSA_OK) return s;
    if ((s = check_dims(B, T, Nmax)) != MSA_OK) return s;
    if (B == 0 || T == 0) return MSA_OK;
    if ((int64_t)B * T * cfg->num_kv_groups > ((int64_t)1 << 31) - 1)
        return fail(MSA_ERR_UNSUPPORTED, "B*T*G exceeds 2^31-1 rows");
    if (!q_idx || !k_idx || !kv_lens || !sel)
        return fail(MSA_ERR_INVALID_ARG, "q_idx, k_idx, kv_lens and sel must not be NULL");
    if (!aligned(q_idx, 16) || !aligned(k_idx, 16))
        return fail(MSA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
    if (!aligned(kv_lens, 4) || (q_start && !aligned(q_start, 4)) || !aligned(sel, 4) ||
        (sel_scores && !aligned(sel_scores, 4)))
        return fail(MSA_ERR_INVALID_ARG, "int32/fp32 arrays must be 4-byte aligned");
    return check_ws(workspace, ws_bytes, index_ws(cfg, B, T, Nmax).total);
}

msa_status check_pool_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                           const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                           const int32_t *q_start, const float *pooled) {
    msa_status s = check_config(cfg);
    if (s != MSA_OK) return s;
    if ((s = check_dims(B, T, Nmax)) != MSA_OK) return s;
    if (B == 0 || T == 0) return MSA_OK;
    if ((int64_t)B * T * cfg->num_kv_groups > ((int64_t)1 << 31) - 1)
        return fail(MSA_ERR_UNSUPPORTED, "B*T*G exceeds 2^31-1 rows");
    if (!q_idx || !k_idx || !kv_lens || !pooled)
        return fail(MSA_ERR_INVALID_ARG, "q_idx, k_idx, kv_lens and pooled must not be NULL");
    if (!aligned(q_idx, 16) || !aligned(k_idx, 16))
        return fail(MSA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
    if (!aligned(kv_lens, 4) || (q_start && !aligned(q_start, 4)) || !aligned(pooled, 4))
        return fail(MSA_ERR_INVALID_ARG, "int32/fp32 arrays must be 4-byte aligned");
    return MSA_OK;
}

int32_t qblock_slots(int32_t T) { return T <= 0 ? 0 : (T - 1 + kBlock - 1) / kBlock + 1; }

msa_status check_qblock_index_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                   const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                                   const int32_t *q_start, const int32_t *sel,
                                   const float *sel_scores) {
    msa_status s = check_config(cfg);
    if (s != MSA_OK) return s;
    if (cfg->topk > kPrefillRegTopk)
        return fail(MSA_ERR_UNSUPPORTED,
                    "query-block selection keeps its top-K in registers: topk %d above %d",
                    cfg->topk, kPrefillRegTopk);
    if ((s = check_dims(B, T, Nmax)) != MSA_OK) return s;
    if (B == 0 || T == 0) return MSA_OK;
    if ((int64_t)B * T * cfg->num_kv_groups > ((int64_t)1 << 31) - 1)
        return fail(MSA_ERR_UNSUPPORTED, "B*T*G exceeds 2^31-1 rows");
    if (!q_idx || !k_idx || !kv_lens || !sel)
        return fail(MSA_ERR_INVALID_ARG, "q_idx, k_idx, kv_lens and sel must not be NULL");
    if (!aligned(q_idx, 16) || !aligned(k_idx, 16))
        return fail(MSA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
    if (!aligned(kv_lens, 4) || (q_start && !aligned(q_start, 4)) || !aligned(sel, 4) ||
        (sel_scores && !aligned(sel_scores, 4)))
        return fail(MSA_ERR_INVALID_ARG, "int32/fp32 arrays must be 4-byte aligned");
    return MSA_OK;
}

msa_status check_backward_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                               const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *kv_lens, const int32_t *q_start,
                               const int32_t *sel, const void *out, const float *lse,
                               const void *dout, const float *dq, const float *dk,
                               const float *dv, const void *workspace, size_t ws_bytes) {
    msa_status s = check_config(cfg);
    if (s != MSA_OK) return s;
    if ((s = check_dims(B, T, Nmax)) != MSA_OK) return s;
    if (B == 0 || T == 0) return MSA_OK;
    const PrefillWs pw = prefill_ws(cfg, B, T, Nmax, true);
    if (pw.nlists + 1 > ((int64_t)1 << 31) - 1 ||
        pw.nslots * cfg->heads_per_group > ((int64_t)1 << 31) - 1 ||
        pw.max_tiles >= ((int64_t)1 << 24))
        return fail(MSA_ERR_UNSUPPORTED, "sparse backward lists exceed 2^31 entries");
    if (!q || !k_cache || !v_cache || !kv_lens || !sel || !out || !lse || !dout || !dq || !dk ||
        !dv)
        return fail(MSA_ERR_INVALID_ARG,
                    "q, k_cache, v_cache, kv_lens, sel, out, lse, dout, dq, dk and dv must not "
                    "be NULL");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
        !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return fail(MSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (!aligned(kv_lens, 4) || (q_start && !aligned(q_start, 4)) || !aligned(sel, 4) ||
        !aligned(lse, 4))
        return fail(MSA_ERR_INVALID_ARG, "int32/fp32 arrays must be 4-byte aligned");
    return check_ws(workspace, ws_bytes, pw.total);
}

msa_status check_project_args(const msa_config *cfg, int32_t M, int32_t hidden_dim,
                              const void *hidden, const void *w, const void *q_idx,
                              const void *k_idx) {
    msa_status s = check_config(cfg);
    if (s != MSA_OK) return s;
    if (cfg->index_dtype != MSA_BF16)
        return fail(MSA_ERR_UNSUPPORTED,
                    "index projections write bf16 index data (index_dtype must be MSA_BF16)");
    if (M < 0) return fail(MSA_ERR_INVALID_ARG, "M must be >= 0");
    if (hidden_dim < 64 || hidden_dim % 64 != 0)
        return fail(MSA_ERR_UNSUPPORTED, "hidden_dim %d unsupported (need a multiple of 64)",
                    hidden_dim);
    if (M == 0) return MSA_OK;
    if (!hidden || !w || !q_idx)
        return fail(MSA_ERR_INVALID_ARG, "hidden, w and q_idx must not be NULL");
    if (!aligned(hidden, 16) || !aligned(w, 16) || !aligned(q_idx, 16) ||
        (k_idx && !aligned(k_idx, 16)))
        return fail(MSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    return MSA_OK;
}

msa_status check_append_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                             const void *k_new, const void *v_new, const void *k_idx_new,
                             const int32_t *pos0, const void *k_cache, const void *v_cache,
                             const void *k_idx) {
    msa_status s = check_config(cfg);
    if (s != MSA_OK) return s;
    if ((s = check_dims(B, T, Nmax)) != MSA_OK) return s;
    if (B == 0 || T == 0) return MSA_OK;
    if ((int64_t)B * T > ((int64_t)1 << 31) - 1)
        return fail(MSA_ERR_UNSUPPORTED, "B*T exceeds 2^31-1 rows");
    if (!k_new || !v_new || !k_idx_new || !pos0 || !k_cache || !v_cache || !k_idx)
        return fail(MSA_ERR_INVALID_ARG,
                    "k_new, v_new, k_idx_new, pos0, k_cache, v_cache and k_idx must not be NULL");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_idx_new, 16) ||
        !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_idx, 16))
        return fail(MSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (!aligned(pos0, 4)) return fail(MSA_ERR_INVALID_ARG, "pos0 must be 4-byte aligned");
    return MSA_OK;
}

msa_status check_sparse_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                             const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *kv_lens, const int32_t *q_start, const int32_t *sel,
                             const void *out, const float *lse, const void *workspace,
                             size_t ws_bytes, int32_t which) {
    msa_status s = check_config(cfg);
    if (s != MSA_OK) return s;
    if ((s = check_dims(B, T, Nmax)) != MSA_OK) return s;
    if (B == 0 || T == 0) return MSA_OK;
    if ((int64_t)B * T * cfg->num_kv_groups * decode_splits(cfg, B) > ((int64_t)1 << 31) - 1)
        return fail(MSA_ERR_UNSUPPORTED, "too many (row, group) work items");
    if (which == MSA_WS_SPARSE_PREFILL) {
        const PrefillWs pw = prefill_ws(cfg, B, T, Nmax);
        if (pw.kv_major && (pw.nlists + 1 > ((int64_t)1 << 31) - 1 ||
                            pw.nslots * cfg->heads_per_group > ((int64_t)1 << 31) - 1 ||
                            pw.max_tiles >= ((int64_t)1 << 24)))
            return fail(MSA_ERR_UNSUPPORTED, "sparse prefill lists exceed 2^31 entries");
    }
    if (!q || !k_cache || !v_cache || !kv_lens || !sel || !out)
        return fail(MSA_ERR_INVALID_ARG, "q, k_cache, v_cache, kv_lens, sel and out must not be NULL");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return fail(MSA_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (!aligned(kv_lens, 4) || (q_start && !aligned(q_start, 4)) || !aligned(sel, 4) ||
        (lse && !aligned(lse, 4)))
        return fail(MSA_ERR_INVALID_ARG, "int32/fp32 arrays must be 4-byte aligned");
    if (which < 0) return MSA_OK;  // a call without workspace
    if (which == MSA_WS_SPARSE_DECODE)
        return check_ws(workspace, ws_bytes, decode_ws(cfg, B, Nmax, false).total);
    return check_ws(workspace, ws_bytes, prefill_ws(cfg, B, T, Nmax).total);
}

msa_status check_decode_args(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                             const void *q_idx, const void *k_idx, const void *k_cache,
                             const void *v_cache, const int32_t *kv_lens, const int32_t *sel,
                             const float *sel_scores, const void *out, const float *lse,
                             const void *workspace, size_t ws_bytes) {
    msa_status s = check_decode_shapes(cfg, B, Nmax, q, q_idx, k_idx, k_cache, v_cache, kv_lens,
                                       sel, sel_scores, out, lse);
    if (s != MSA_OK || B == 0) return s;
    return check_ws(workspace, ws_bytes, decode_ws(cfg, B, Nmax, true).total);
}

msa_status check_decode_shapes(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                               const void *q_idx, const void *k_idx, const void *k_cache,
                               const void *v_cache, const int32_t *kv_lens, const int32_t *sel,
                               const float *sel_scores, const void *out, const float *lse) {
    msa_status s = check_config(cfg);
    if (s != MSA_OK) return s;
    if ((s = check_dims(B, 1, Nmax)) != MSA_OK) return s;
    if (B == 0) return MSA_OK;
    if ((int64_t)B * cfg->num_kv_groups > ((int64_t)1 << 31) - 1)
        return fail(MSA_ERR_UNSUPPORTED, "too many (sequence, group) work items");
    if (!q || !q_idx || !k_idx || !k_cache || !v_cache || !kv_lens || !sel || !out)
        return fail(MSA_ERR_INVALID_ARG,
                    "q, q_idx, k_idx, k_cache, v_cache, kv_lens, sel and out must not be NULL");
    if (!aligned(q, 16) || !aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(out, 16))
        return fail(MSA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (!aligned(kv_lens, 4) || !aligned(sel, 4) || (sel_scores && !aligned(sel_scores, 4)) ||
        (lse && !aligned(lse, 4)))
        return fail(MSA_ERR_INVALID_ARG, "int32/fp32 arrays must be 4-byte aligned");
    return MSA_OK;
}

}  // namespace msa

extern "C" {

size_t msa_workspace_size(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                          int32_t which) {
    if (msa::check_config(cfg) != MSA_OK || B < 0 || T < 0 || Nmax < 0) return (size_t)-1;
    switch (which) {
        case MSA_WS_INDEX_TOPK:
            return msa::index_ws(cfg, B, T, Nmax).total;
        case MSA_WS_SPARSE_PREFILL:
            return msa::prefill_ws(cfg, B, T, Nmax).total;
        case MSA_WS_SPARSE_DECODE:
            return msa::decode_ws(cfg, B, Nmax, false).total;
        case MSA_WS_DECODE:
            return msa::decode_ws(cfg, B, Nmax, true).total;
        case MSA_WS_SPARSE_BACKWARD:
            return msa::prefill_ws(cfg, B, T, Nmax, true).total;
        default:
            msa::fail(MSA_ERR_INVALID_ARG, "unknown workspace kind %d", which);
            return (size_t)-1;
    }
}

const char *msa_status_string(msa_status s) {
    switch (s) {
        case MSA_OK: return "MSA_OK";
        case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
        case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
        case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
        case MSA_ERR_HIP: return "MSA_ERR_HIP";
    }
    return "MSA_ERR_UNKNOWN";
}

const char *msa_last_error(void) { return msa::g_err; }

int32_t msa_version(void) { return 100; }

int32_t msa_qblock_slots(int32_t T) { return msa::qblock_slots(T); }

}  // extern "C"

// Private interface between the host-only validation unit (msa_host.cpp) and
// the kernel units (msa_decode.hip, msa_prefill.hip, msa_backward.hip). Not
// installed; not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

constexpr int kHeadDim = 128;
constexpr int kIndexDim = 128;
constexpr int kBlock = 128;
constexpr int kMaxTopk = 64;
// The prefill index kernel keeps a row's top-K in registers up to this K;
// above it msa_index_topk writes pooled scores to the workspace and ranks
// them per row (the decode path's ranking).
constexpr int kPrefillRegTopk = 32;
constexpr int kMaxHeadsPerGroup = 16;
constexpr int kScanMaxRows = 16;  // T*G at or below this uses the streaming index kernel
// The MFMA prefill index kernel takes kIdxTileRows (row, group) rows of one
// sequence per workgroup. With fewer than kIdxRegMinWgs such workgroups (a
// short prefill) msa_index_topk splits every tile's key blocks over several
// workgroups instead, writing pooled scores, and ranks the rows afterwards.
constexpr int kIdxTileRows = 256;
constexpr int64_t kIdxRegMinWgs = 64;
// msa_index_topk's path: pooled scores in the workspace, then a wavefront per
// row ranks them (decode shapes, K above the register top-K, short
// prefills); otherwise the prefill kernel ranks each row in registers.
bool index_uses_pooled(const msa_config *cfg, int32_t B, int32_t T);
constexpr size_t kWsAlign = 256;


// Records a formatted message for msa_last_error() on this thread and returns s.
msa_status fail(msa_status s, const char *fmt, ...);
void clear_error();

// Host-side argument checks; each returns MSA_OK or records why not.
msa_status check_config(const msa_config *cfg);
msa_status check_index_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                            const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                            const int32_t *q_start, const int32_t *sel, const float *sel_scores,
                            const void *workspace, size_t ws_bytes);
msa_status check_pool_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                           const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                           const int32_t *q_start, const float *pooled);
msa_status check_project_args(const msa_config *cfg, int32_t M, int32_t hidden_dim,
                              const void *hidden, const void *w, const void *q_idx,
                              const void *k_idx);
msa_status check_append_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                             const void *k_new, const void *v_new, const void *k_idx_new,
                             const int32_t *pos0, const void *k_cache, const void *v_cache,
                             const void *k_idx);
int32_t qblock_slots(int32_t T);
msa_status check_qblock_index_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                   const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                                   const int32_t *q_start, const int32_t *sel,
                                   const float *sel_scores);
msa_status check_backward_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                               const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *kv_lens, const int32_t *q_start,
                               const int32_t *sel, const void *out, const float *lse,
                               const void *dout, const float *dq, const float *dk,
                               const float *dv, const void *workspace, size_t ws_bytes);
msa_status check_sparse_args(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                             const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *kv_lens, const int32_t *q_start, const int32_t *sel,
                             const void *out, const float *lse, const void *workspace,
                             size_t ws_bytes, int32_t which);

// Workspace layout: when index_uses_pooled (and in msa_decode) the index
// branch keeps the pooled block scores of every row, [B*T*G][ceil(Nmax/S)]
// fp32; the register top-K path needs none.
struct IndexWs {
    size_t pooled_off, pooled_bytes, total;
    int64_t nb_max;  // ceil(Nmax / S)
};
IndexWs index_ws(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax);

// Sparse prefill. Below kPfKvMajorMinRows (B*T*G) rows the query-major kernel
// runs (no workspace). Otherwise the KV-major path works in passes over
// `groups` groups and `rows` query rows of every sequence (see prefill_ws). Per pass the workspace holds the
// per-(sequence, group, block) row bitmaps with their word prefix counts,
// list sizes, offsets and tile starts, the tile -> list map, the lists, and
// per-(row, group, slot, head) partials: O / l in bf16 [d] and (m, l) as two
// fp32.
constexpr int64_t kPfKvMajorMinRows = 256;
constexpr size_t kPfPartialBudget = (size_t)5 << 30;
constexpr size_t kPfBitmapBudget = (size_t)1 << 30;
constexpr int kPfWaves = 4;       // waves per attention workgroup
constexpr int kPfNq = 2;          // 16-column query tiles per wave
constexpr int kPfRounds = 16;     // passes of every wave over its tiles per workgroup
constexpr int64_t kPfFillTiles = 1024;  // fewer rounds per tile below this many tiles a pass
int32_t prefill_entries_per_tile(int32_t R);
struct PrefillWs {
    bool kv_major;
    int32_t rows;    // query rows of every sequence per pass
    int32_t groups;  // groups per pass
    int32_t entries_per_tile;
    int64_t nb_max, nlists, nslots, max_tiles;
    int32_t bit_words;  // 32-bit words of a list's row bitmap: ceil(rows / 32)
    size_t bits_off, wpre_off, counts_off, offsets_off, tile_first_off, tile_map_off, list_off;
    size_t part_o_off, part_ml_off, delta_off;
    // Target of the stores of columns that hold no entry (their values are
    // discarded), so the attention kernels store unconditionally.
    size_t trash_off;
    size_t total;
};
constexpr size_t kPfTrashBytes = 8192;  // >= one entry's R*d bf16 values and R (m, l) pairs
// backward: the layout of msa_sparse_attn_backward (always KV-major; dq
// partials in bf16 instead of the forward's partials; plus dout.out per
// (row, head)).
PrefillWs prefill_ws(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                     bool backward = false);

// Decode attention: split partials [B*G][nsplit][R] x (128 + 2) fp32, after
// the pooled scores when the call also runs the index branch (msa_decode).
// A split is one workgroup of decode_waves(cfg, B) waves, one 32-token chunk
// each: 16 waves when the (sequence, group, split) grid of 16-wave
// workgroups has at least kDecodeFillWorkgroups of them, else 8 (more, smaller
// workgroups for few sequences).
constexpr int64_t kDecodeFillWorkgroups = 256;
int32_t decode_waves(const msa_config *cfg, int32_t B);
int32_t decode_splits(const msa_config *cfg, int32_t B);
// msa_decode also keeps one arrival counter per (sequence, group), zeroed by
// the index kernel of the same call.
struct DecodeWs {
    size_t pooled_off, part_o_off, part_ml_off, counters_off, total;
    int64_t nb_max;
};
DecodeWs decode_ws(const msa_config *cfg, int32_t B, int32_t Nmax, bool with_index);

// check_decode_args without the workspace (msa_decode_no_alloc).
msa_status check_decode_shapes(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                               const void *q_idx, const void *k_idx, const void *k_cache,
                               const void *v_cache, const int32_t *kv_lens, const int32_t *sel,
                               const float *sel_scores, const void *out, const float *lse);
msa_status check_decode_args(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                             const void *q_idx, const void *k_idx, const void *k_cache,
                             const void *v_cache, const int32_t *kv_lens, const int32_t *sel,
                             const float *sel_scores, const void *out, const float *lse,
                             const void *workspace, size_t ws_bytes);

}  // namespace msa

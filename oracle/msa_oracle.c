/*
 * CPU oracle for MiniMax Sparse Attention (MSA) — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 statement of the method, written row by row so that
 * any single query row can be checked on its own. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load this library; it
 * shares no code with the GPU kernels.
 *
 * Pages followed (MiniMax M3 sparse attention articles):
 *   [T] cloud.tencent.com, "Something BIG Is Coming 百万token上下文提速近10倍，
 *       MiniMax M3的稀疏注意力凭什么这么快", §二 and §六;
 *   [M] mlqm.cn, "如何用MiniMax-M3的稀疏注意力技术解决大模型效率瓶颈",
 *       section 核心原理 (sparse_attention_config).
 *
 * Readings where the pages are silent (each is stated once here and next to
 * the code that depends on it):
 *   - the index score is the plain dot product of the group's index query
 *     with the token's index key (no scale, no activation);
 *   - one index key per token, shared by every group;
 *   - selection is per query token and per group (the query-block-shared
 *     variant of [M] 核心原理 is oracle_index_topk_qblock, reading stated there);
 *   - causal: a row at position p pools and attends only over keys j <= p;
 *   - fewer valid blocks than K: all valid blocks are kept, then -1 padding;
 *   - no block is forced in (no sink, no local window);
 *   - equal pooled scores: the lower block id ranks first;
 *   - softmax scale 1/sqrt(d) on attention logits; index scores unscaled;
 *   - query head h belongs to group h / R.
 */
#include "msa_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_value(uint16_t bits) {
    /* bfloat16 is the upper half of an IEEE binary32. */
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)bits << 16;
    return (double)v.f;
}

double oracle_e4m3_value(uint8_t bits) {
    /* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits; no
     * infinities; S.1111.111 is NaN; exponent 0 is subnormal. */
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 15;
    int m = bits & 7;
    double mag;
    if (e == 15 && m == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* The 256 E4M3 values, decoded once by oracle_e4m3_value (a lookup keeps
 * long rows fast; the values are the decoder's own). */
static double e4m3_table[256];
static pthread_once_t e4m3_once = PTHREAD_ONCE_INIT;

static void fill_e4m3_table(void) {
    for (int c = 0; c < 256; ++c) e4m3_table[c] = oracle_e4m3_value((uint8_t)c);
}

static double index_elem(const oracle_cfg *cfg, const void *base, int64_t i) {
    if (cfg->index_dtype == 1) {
        pthread_once(&e4m3_once, fill_e4m3_table);
        return e4m3_table[((const uint8_t *)base)[i]];
    }
    return oracle_bf16_value(((const uint16_t *)base)[i]);
}

static int check_cfg(const oracle_cfg *c) {
    if (!c || c->groups < 1 || c->heads_per_group < 1 || c->head_dim < 1 || c->index_dim < 1 ||
        c->block_size < 1 || c->topk < 1 || (c->index_dtype != 0 && c->index_dtype != 1))
        return -1;
    return 0;
}

typedef struct {
    double score;
    int32_t block;
} ranked_block;

/* Total order of [T] §二's top-k: higher pooled score first, then lower id. */
static int rank_cmp(const void *a, const void *b) {
    const ranked_block *x = a, *y = b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->block > y->block) - (x->block < y->block);
}

/* [T] §二, first two steps: the index query of group g scored against every
 * past index key, then max-pooled over each block. */
int oracle_index_pool_row(const oracle_cfg *cfg, const void *q_idx_row, const void *k_idx_seq,
                          int64_t p, double *pooled) {
    if (check_cfg(cfg) || p < 0 || !q_idx_row || !k_idx_seq || !pooled) return -1;
    const int G = cfg->groups, dI = cfg->index_dim, S = cfg->block_size;
    const int64_t n_valid = p / S + 1; /* blocks holding at least one key j <= p */
    double *s = malloc(sizeof(double) * (size_t)(p + 1));
    if (!s) return -1;
    for (int g = 0; g < G; ++g) {
        /* Step 1: s_j = sum_c q_I[g, c] * k_I[j, c] for every j <= p. */
        for (int64_t j = 0; j <= p; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dI; ++c)
                acc += index_elem(cfg, q_idx_row, (int64_t)g * dI + c) *
                       index_elem(cfg, k_idx_seq, j * dI + c);
            s[j] = acc;
        }
        /* Step 2: causal block max-pool; block beta covers
         * [beta*S, min(beta*S + S - 1, p)]. */
        for (int64_t beta = 0; beta < n_valid; ++beta) {
            int64_t lo = beta * S, hi = beta * S + S - 1;
            if (hi > p) hi = p;
            double m = s[lo];
            for (int64_t j = lo + 1; j <= hi; ++j)
                if (s[j] > m) m = s[j];
            pooled[g * n_valid + beta] = m;
        }
    }
    free(s);
    return 0;
}

/* [T] §二, third step: of the pooled scores, the top-K blocks are kept. */
int oracle_index_topk_row(const oracle_cfg *cfg, const void *q_idx_row, const void *k_idx_seq,
                          int64_t p, int32_t *sel, double *scores) {
    if (check_cfg(cfg) || p < 0 || !q_idx_row || !k_idx_seq || !sel) return -1;
    const int G = cfg->groups, S = cfg->block_size, K = cfg->topk;
    const int64_t n_valid = p / S + 1;
    double *pooled = malloc(sizeof(double) * (size_t)(G * n_valid));
    ranked_block *pool = malloc(sizeof(ranked_block) * (size_t)n_valid);
    if (!pooled || !pool || oracle_index_pool_row(cfg, q_idx_row, k_idx_seq, p, pooled)) {
        free(pooled);
        free(pool);
        return -1;
    }
    for (int g = 0; g < G; ++g) {
        for (int64_t beta = 0; beta < n_valid; ++beta) {
            pool[beta].score = pooled[g * n_valid + beta];
            pool[beta].block = (int32_t)beta;
        }
        /* Order all valid blocks, keep the first min(K, n_valid). */
        qsort(pool, (size_t)n_valid, sizeof(ranked_block), rank_cmp);
        for (int k = 0; k < K; ++k) {
            if (k < n_valid) {
                sel[g * K + k] = pool[k].block;
                if (scores) scores[g * K + k] = pool[k].score;
            } else {
                sel[g * K + k] = -1;
                if (scores) scores[g * K + k] = -INFINITY;
            }
        }
    }
    free(pooled);
    free(pool);
    return 0;
}

/* Query-block-shared selection ([M] 核心原理: the sequence is cut into
 * 128-token blocks and each block interacts with its 16 most relevant
 * blocks). Reading: the query block of a row at position p is p / S (the
 * same blocks as the keys); for the rows of one query block that the call
 * holds, a key block's score is the largest pooled score any of those rows
 * gives it (each row pooling causally, as in oracle_index_pool_row), and the
 * top-K of those scores, in the order of rank_cmp, is shared by every row of
 * the block. q_idx_seq [T, G, d_I] holds this sequence's rows, row i at
 * position q_start + i; rows at or past kv_len do not exist. `slot` counts
 * query blocks from q_start's block. Writes sel[G*K] and scores[G*K] (-1 /
 * -inf when the block has no row). */
int oracle_index_topk_qblock(const oracle_cfg *cfg, const void *q_idx_seq, int32_t T,
                             const void *k_idx_seq, int64_t q_start, int64_t kv_len,
                             int64_t slot, int32_t *sel, double *scores) {
    if (check_cfg(cfg) || T < 0 || q_start < 0 || slot < 0 || !q_idx_seq || !k_idx_seq || !sel)
        return -1;
    const int G = cfg->groups, dI = cfg->index_dim, S = cfg->block_size, K = cfg->topk;
    const int64_t qb = q_start / S + slot;
    const int64_t es = cfg->index_dtype == 1 ? 1 : 2;
    /* Rows of the call in query block qb (positions below kv_len). */
    int64_t i_lo = qb * S - q_start, i_hi = qb * S + S - 1 - q_start;
    if (i_lo < 0) i_lo = 0;
    if (i_hi > T - 1) i_hi = T - 1;
    if (i_hi > kv_len - 1 - q_start) i_hi = kv_len - 1 - q_start;
    for (int k = 0; k < G * K; ++k) {
        sel[k] = -1;
        if (scores) scores[k] = -INFINITY;
    }
    if (i_lo > i_hi) return 0;
    const int64_t n_valid = (q_start + i_hi) / S + 1; /* = qb + 1 */
    double *best = malloc(sizeof(double) * (size_t)(G * n_valid));
    double *row = malloc(sizeof(double) * (size_t)(G * n_valid));
    ranked_block *pool = malloc(sizeof(ranked_block) * (size_t)n_valid);
    if (!best || !row || !pool) {
        free(best);
        free(row);
        free(pool);
        return -1;
    }
    for (int64_t k = 0; k < G * n_valid; ++k) best[k] = -INFINITY;
    for (int64_t i = i_lo; i <= i_hi; ++i) {
        const int64_t p = q_start + i;
        const int64_t nv = p / S + 1;
        const char *qrow = (const char *)q_idx_seq + i * G * dI * es;
        if (oracle_index_pool_row(cfg, qrow, k_idx_seq, p, row)) {
            free(best);
            free(row);
            free(pool);
            return -1;
        }
        for (int g = 0; g < G; ++g)
            for (int64_t beta = 0; beta < nv; ++beta)
                if (row[g * nv + beta] > best[g * n_valid + beta])
                    best[g * n_valid + beta] = row[g * nv + beta];
    }
    for (int g = 0; g < G; ++g) {
        for (int64_t beta = 0; beta < n_valid; ++beta) {
            pool[beta].score = best[g * n_valid + beta];
            pool[beta].block = (int32_t)beta;
        }
        qsort(pool, (size_t)n_valid, sizeof(ranked_block), rank_cmp);
        for (int k = 0; k < K && k < n_valid; ++k) {
            sel[g * K + k] = pool[k].block;
            if (scores) scores[g * K + k] = pool[k].score;
        }
    }
    free(best);
    free(row);
    free(pool);
    return 0;
}

static double tau_of(const oracle_cfg *cfg) {
    return cfg->softmax_scale > 0 ? cfg->softmax_scale : 1.0 / sqrt((double)cfg->head_dim);
}

/* Softmax attention of one head over the key positions listed in keys[0..n). */
static void attend(const oracle_cfg *cfg, const uint16_t *q_head, const uint16_t *k_grp,
                   const uint16_t *v_grp, const int64_t *keys, int64_t n, double *z,
                   double *out_head, double *lse_head) {
    const int d = cfg->head_dim;
    const double tau = tau_of(cfg);
    double m = -INFINITY;
    for (int64_t a = 0; a < n; ++a) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
            acc += oracle_bf16_value(q_head[c]) * oracle_bf16_value(k_grp[keys[a] * d + c]);
        z[a] = tau * acc;
        if (z[a] > m) m = z[a];
    }
    double l = 0.0;
    for (int64_t a = 0; a < n; ++a) l += exp(z[a] - m);
    for (int c = 0; c < d; ++c) out_head[c] = 0.0;
    for (int64_t a = 0; a < n; ++a) {
        double w = exp(z[a] - m) / l;
        for (int c = 0; c < d; ++c) out_head[c] += w * oracle_bf16_value(v_grp[keys[a] * d + c]);
    }
    if (lse_head) *lse_head = m + log(l);
}

/* [T] §二 sparse branch + §六 GQA sharing: every head of group g attends over
 * J = { j <= p : block(j) in sel[g] }. */
int oracle_sparse_attn_row(const oracle_cfg *cfg, const uint16_t *q_row, const uint16_t *k_seq,
                           const uint16_t *v_seq, int64_t n_stride, int64_t p,
                           const int32_t *sel, double *out, double *lse) {
    if (check_cfg(cfg) || p < 0 || p >= n_stride || !q_row || !k_seq || !v_seq || !sel || !out)
        return -1;
    const int G = cfg->groups, R = cfg->heads_per_group, d = cfg->head_dim;
    const int S = cfg->block_size, K = cfg->topk;
    const int64_t n_valid = p / S + 1;
    char *chosen = malloc((size_t)n_valid);
    int64_t *keys = malloc(sizeof(int64_t) * (size_t)(p + 1));
    double *z = malloc(sizeof(double) * (size_t)(p + 1));
    if (!chosen || !keys || !z) {
        free(chosen);
        free(keys);
        free(z);
        return -1;
    }
    for (int g = 0; g < G; ++g) {
        memset(chosen, 0, (size_t)n_valid);
        for (int k = 0; k < K; ++k) {
            int32_t b = sel[g * K + k];
            if (b >= 0 && b < n_valid) chosen[b] = 1;
        }
        int64_t n = 0;
        for (int64_t blk = 0; blk < n_valid; ++blk)
            if (chosen[blk])
                for (int64_t j = blk * S; j <= p && j < (blk + 1) * S; ++j) keys[n++] = j;
        const uint16_t *k_grp = k_seq + (int64_t)g * n_stride * d;
        const uint16_t *v_grp = v_seq + (int64_t)g * n_stride * d;
        for (int r = 0; r < R; ++r) {
            int h = g * R + r;
            if (n == 0) { /* nothing to attend to: defined as zero output, lse = -inf */
                for (int c = 0; c < d; ++c) out[(int64_t)h * d + c] = 0.0;
                if (lse) lse[h] = -INFINITY;
                continue;
            }
            attend(cfg, q_row + (int64_t)h * d, k_grp, v_grp, keys, n, z, out + (int64_t)h * d,
                   lse ? lse + h : NULL);
        }
    }
    free(chosen);
    free(keys);
    free(z);
    return 0;
}

/* Textbook causal GQA softmax attention over all keys j <= p. */
int oracle_dense_causal_row(const oracle_cfg *cfg, const uint16_t *q_row, const uint16_t *k_seq,
                            const uint16_t *v_seq, int64_t n_stride, int64_t p,
                            double *out, double *lse) {
    if (check_cfg(cfg) || p < 0 || p >= n_stride || !q_row || !k_seq || !v_seq || !out)
        return -1;
    const int G = cfg->groups, R = cfg->heads_per_group, d = cfg->head_dim;
    int64_t *keys = malloc(sizeof(int64_t) * (size_t)(p + 1));
    double *z = malloc(sizeof(double) * (size_t)(p + 1));
    if (!keys || !z) {
        free(keys);
        free(z);
        return -1;
    }
    for (int64_t j = 0; j <= p; ++j) keys[j] = j;
    for (int h = 0; h < G * R; ++h) {
        int g = h / R;
        attend(cfg, q_row + (int64_t)h * d, k_seq + (int64_t)g * n_stride * d,
               v_seq + (int64_t)g * n_stride * d, keys, p + 1, z, out + (int64_t)h * d,
               lse ? lse + h : NULL);
    }
    free(keys);
    free(z);
    return 0;
}

/* Backward of the sparse branch. [T] §五 presents the two-branch design as
 * trainable end to end; the selection is a discrete choice and carries no
 * gradient, so for fixed selections the sparse branch is softmax attention
 * over the kept keys and its gradients are the textbook ones. For sequence b
 * and group g, every row i of the call at position p = q_start + i < kv_len,
 * each head h of g, with J the row's attended keys and dout the upstream
 * gradient of out:
 *   P_j = softmax_j(tau q.k_j),  dP_j = dout.v_j,
 *   dS_j = P_j (dP_j - sum_k P_k dP_k),
 *   dq = tau sum_j dS_j k_j,  dk_j += tau dS_j q,  dv_j += P_j dout.
 * q_seq, dout_seq [T, H, d] and k_grp, v_grp [n_stride, d] are bf16 bits;
 * sel_seq [T, G, K]. Writes dq_seq [T, H, d] (heads of group g; zero for rows
 * outside the cache or with nothing to attend to) and dk_grp, dv_grp
 * [n_stride, d] (zero where no row attends). */
int oracle_sparse_attn_backward_group(const oracle_cfg *cfg, int32_t T, int64_t n_stride,
                                      const uint16_t *q_seq, const uint16_t *k_grp,
                                      const uint16_t *v_grp, int64_t kv_len, int64_t q_start,
                                      int32_t g, const int32_t *sel_seq, const uint16_t *dout_seq,
                                      double *dq_seq, double *dk_grp, double *dv_grp) {
    if (check_cfg(cfg) || T < 0 || kv_len > n_stride || g < 0 || g >= cfg->groups || !q_seq ||
        !k_grp || !v_grp || !sel_seq || !dout_seq || !dq_seq || !dk_grp || !dv_grp)
        return -1;
    const int G = cfg->groups, R = cfg->heads_per_group, d = cfg->head_dim;
    const int S = cfg->block_size, K = cfg->topk, H = G * R;
    const double tau = tau_of(cfg);
    for (int64_t x = 0; x < n_stride * d; ++x) dk_grp[x] = dv_grp[x] = 0.0;
    const int64_t nmax = kv_len > 0 ? kv_len : 1;
    char *chosen = malloc((size_t)(nmax / S + 1));
    int64_t *keys = malloc(sizeof(int64_t) * (size_t)nmax);
    double *P = malloc(sizeof(double) * (size_t)nmax);
    double *dP = malloc(sizeof(double) * (size_t)nmax);
    if (!chosen || !keys || !P || !dP) {
        free(chosen);
        free(keys);
        free(P);
        free(dP);
        return -1;
    }
    for (int32_t i = 0; i < T; ++i) {
        const int64_t p = q_start + i;
        for (int r = 0; r < R; ++r)
            for (int c = 0; c < d; ++c) dq_seq[((int64_t)i * H + g * R + r) * d + c] = 0.0;
        if (p < 0 || p >= kv_len) continue;
        const int64_t n_valid = p / S + 1;
        memset(chosen, 0, (size_t)n_valid);
        for (int k = 0; k < K; ++k) {
            const int32_t blk = sel_seq[((int64_t)i * G + g) * K + k];
            if (blk >= 0 && blk < n_valid) chosen[blk] = 1;
        }
        int64_t n = 0;
        for (int64_t blk = 0; blk < n_valid; ++blk)
            if (chosen[blk])
                for (int64_t j = blk * S; j <= p && j < (blk + 1) * S; ++j) keys[n++] = j;
        if (n == 0) continue;
        for (int r = 0; r < R; ++r) {
            const int64_t h = g * R + r;
            const uint16_t *qh = q_seq + ((int64_t)i * H + h) * d;
            const uint16_t *doh = dout_seq + ((int64_t)i * H + h) * d;
            double m = -INFINITY;
            for (int64_t a = 0; a < n; ++a) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c)
                    acc += oracle_bf16_value(qh[c]) * oracle_bf16_value(k_grp[keys[a] * d + c]);
                P[a] = tau * acc;
                if (P[a] > m) m = P[a];
            }
            double l = 0.0;
            for (int64_t a = 0; a < n; ++a) {
                P[a] = exp(P[a] - m);
                l += P[a];
            }
            double delta = 0.0;
            for (int64_t a = 0; a < n; ++a) {
                P[a] /= l;
                double acc = 0.0;
                for (int c = 0; c < d; ++c)
                    acc += oracle_bf16_value(doh[c]) * oracle_bf16_value(v_grp[keys[a] * d + c]);
                dP[a] = acc;
                delta += P[a] * acc;
            }
            double *dqh = dq_seq + ((int64_t)i * H + h) * d;
            for (int64_t a = 0; a < n; ++a) {
                const double ds = P[a] * (dP[a] - delta);
                const int64_t j = keys[a];
                for (int c = 0; c < d; ++c) {
                    dqh[c] += tau * ds * oracle_bf16_value(k_grp[j * d + c]);
                    dk_grp[j * d + c] += tau * ds * oracle_bf16_value(qh[c]);
                    dv_grp[j * d + c] += P[a] * oracle_bf16_value(doh[c]);
                }
            }
        }
    }
    free(chosen);
    free(keys);
    free(P);
    free(dP);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Row-parallel drivers: a pthread pool pulling row numbers from a counter.   */

typedef struct {
    int kind; /* 0 index, 1 sparse, 2 dense, 3 pooled, 4 query-block index, 5 backward */
    const oracle_cfg *cfg;
    int32_t T;
    int64_t n_stride;
    const void *q_idx, *k_idx;
    const uint16_t *q, *k_cache, *v_cache;
    const int32_t *kv_lens, *q_start, *rows_b, *rows_i, *sel_in;
    int64_t nrows;
    int32_t *sel;
    double *scores, *out, *lse, *pooled;
    const uint16_t *dout; /* backward: upstream gradient; out holds dq */
    double *dk, *dv;
    int64_t nb_out; /* pooled: blocks stored per (row, group) */
    int64_t next; /* shared row counter */
    int failed;
} row_work;

static int64_t index_elem_size(const oracle_cfg *cfg) { return cfg->index_dtype == 1 ? 1 : 2; }

static int run_row(row_work *w, int64_t r) {
    const oracle_cfg *cfg = w->cfg;
    const int G = cfg->groups, H = cfg->groups * cfg->heads_per_group;
    const int d = cfg->head_dim, dI = cfg->index_dim, K = cfg->topk;
    int32_t b = w->rows_b[r], i = w->rows_i[r];
    if (b < 0 || i < 0 || (w->kind < 4 && i >= w->T)) return -1;
    int64_t p = (int64_t)w->q_start[b] + i;
    if (w->kind < 4 && (p >= w->kv_lens[b] || w->kv_lens[b] > w->n_stride)) return -1;
    if (w->kind == 5) {
        /* (sequence, group): rows_i holds the group. */
        const int64_t H = (int64_t)G * cfg->heads_per_group;
        if (w->kv_lens[b] > w->n_stride) return -1;
        return oracle_sparse_attn_backward_group(
            cfg, w->T, w->n_stride, w->q + (int64_t)b * w->T * H * d,
            w->k_cache + ((int64_t)b * G + i) * w->n_stride * d,
            w->v_cache + ((int64_t)b * G + i) * w->n_stride * d, w->kv_lens[b], w->q_start[b], i,
            w->sel_in + (int64_t)b * w->T * G * K, w->dout + (int64_t)b * w->T * H * d,
            w->out + (int64_t)b * w->T * H * d,
            w->dk + ((int64_t)b * G + i) * w->n_stride * d,
            w->dv + ((int64_t)b * G + i) * w->n_stride * d);
    }
    if (w->kind == 4) {
        /* (sequence, query-block slot): rows_i holds the slot. */
        const int64_t es = index_elem_size(cfg);
        const char *qseq = (const char *)w->q_idx + ((int64_t)b * w->T * G * dI) * es;
        const char *kseq = (const char *)w->k_idx + ((int64_t)b * w->n_stride * dI) * es;
        if (w->kv_lens[b] > w->n_stride || w->q_start[b] < 0) return -1;
        return oracle_index_topk_qblock(cfg, qseq, w->T, kseq, w->q_start[b], w->kv_lens[b], i,
                                        w->sel + r * G * K, w->scores ? w->scores + r * G * K : NULL);
    }
    if (w->kind == 0 || w->kind == 3) {
        int64_t es = index_elem_size(cfg);
        const char *qrow = (const char *)w->q_idx + (((int64_t)b * w->T + i) * G * dI) * es;
        const char *kseq = (const char *)w->k_idx + ((int64_t)b * w->n_stride * dI) * es;
        if (w->kind == 0)
            return oracle_index_topk_row(cfg, qrow, kseq, p, w->sel + r * G * K,
                                         w->scores ? w->scores + r * G * K : NULL);
        /* pooled[r, g, beta] for beta < nb_out; blocks past p are -inf. */
        const int64_t n_valid = p / cfg->block_size + 1;
        if (n_valid > w->nb_out) return -1;
        double *tmp = malloc(sizeof(double) * (size_t)(G * n_valid));
        if (!tmp) return -1;
        int rc = oracle_index_pool_row(cfg, qrow, kseq, p, tmp);
        for (int g = 0; g < G; ++g)
            for (int64_t beta = 0; beta < w->nb_out; ++beta)
                w->pooled[(r * G + g) * w->nb_out + beta] =
                    beta < n_valid ? tmp[g * n_valid + beta] : -INFINITY;
        free(tmp);
        return rc;
    }
    const uint16_t *qrow = w->q + ((int64_t)b * w->T + i) * H * d;
    const uint16_t *kseq = w->k_cache + (int64_t)b * G * w->n_stride * d;
    const uint16_t *vseq = w->v_cache + (int64_t)b * G * w->n_stride * d;
    double *o = w->out + r * H * d;
    double *l = w->lse ? w->lse + r * H : NULL;
    if (w->kind == 1)
        return oracle_sparse_attn_row(cfg, qrow, kseq, vseq, w->n_stride, p,
                                      w->sel_in + r * G * K, o, l);
    return oracle_dense_causal_row(cfg, qrow, kseq, vseq, w->n_stride, p, o, l);
}

static void *row_thread(void *arg) {
    row_work *w = arg;
    for (;;) {
        int64_t r = __atomic_fetch_add(&w->next, 1, __ATOMIC_RELAXED);
        if (r >= w->nrows) break;
        if (run_row(w, r)) __atomic_store_n(&w->failed, 1, __ATOMIC_RELAXED);
    }
    return NULL;
}

static int run_rows(row_work *w, int32_t nthreads) {
    if (check_cfg(w->cfg) || w->nrows < 0) return -1;
    /* nthreads counts the caller's thread; start nthreads - 1 helpers. */
    int64_t helpers = (int64_t)nthreads - 1;
    if (helpers > 511) helpers = 511;
    if (helpers > w->nrows - 1) helpers = w->nrows - 1;
    if (helpers < 0) helpers = 0;
    nthreads = (int32_t)helpers;
    w->next = 0;
    w->failed = 0;
    pthread_t *tid = malloc(sizeof(pthread_t) * (size_t)(nthreads + 1));
    char *ok = calloc((size_t)nthreads + 1, 1);
    if (!tid || !ok) {
        free(tid);
        free(ok);
        return -1;
    }
    for (int t = 0; t < nthreads; ++t) ok[t] = pthread_create(&tid[t], NULL, row_thread, w) == 0;
    row_thread(w); /* the caller's thread works too */
    for (int t = 0; t < nthreads; ++t)
        if (ok[t]) pthread_join(tid[t], NULL);
    free(tid);
    free(ok);
    return w->failed ? -1 : 0;
}

int oracle_index_topk_rows(const oracle_cfg *cfg, int32_t T, int64_t n_stride, const void *q_idx,
                           const void *k_idx, const int32_t *kv_lens, const int32_t *q_start,
                           int64_t nrows, const int32_t *rows_b, const int32_t *rows_i,
                           int32_t nthreads, int32_t *sel, double *scores) {
    row_work w = { 0 };
    w.kind = 0; w.cfg = cfg; w.T = T; w.n_stride = n_stride; w.q_idx = q_idx; w.k_idx = k_idx;
    w.kv_lens = kv_lens; w.q_start = q_start; w.nrows = nrows; w.rows_b = rows_b;
    w.rows_i = rows_i; w.sel = sel; w.scores = scores;
    return run_rows(&w, nthreads);
}

int oracle_index_topk_qblocks(const oracle_cfg *cfg, int32_t T, int64_t n_stride,
                              const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                              const int32_t *q_start, int64_t nitems, const int32_t *items_b,
                              const int32_t *items_slot, int32_t nthreads, int32_t *sel,
                              double *scores) {
    row_work w = { 0 };
    w.kind = 4; w.cfg = cfg; w.T = T; w.n_stride = n_stride; w.q_idx = q_idx; w.k_idx = k_idx;
    w.kv_lens = kv_lens; w.q_start = q_start; w.nrows = nitems; w.rows_b = items_b;
    w.rows_i = items_slot; w.sel = sel; w.scores = scores;
    return run_rows(&w, nthreads);
}

int oracle_sparse_attn_backward(const oracle_cfg *cfg, int32_t B, int32_t T, int64_t n_stride,
                                const uint16_t *q, const uint16_t *k_cache,
                                const uint16_t *v_cache, const int32_t *kv_lens,
                                const int32_t *q_start, const int32_t *sel, const uint16_t *dout,
                                int32_t nthreads, double *dq, double *dk, double *dv) {
    if (check_cfg(cfg) || B < 0) return -1;
    const int64_t n = (int64_t)B * cfg->groups;
    int32_t *ib = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t *ig = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    if (!ib || !ig) {
        free(ib);
        free(ig);
        return -1;
    }
    for (int64_t x = 0; x < n; ++x) {
        ib[x] = (int32_t)(x / cfg->groups);
        ig[x] = (int32_t)(x % cfg->groups);
    }
    row_work w = { 0 };
    w.kind = 5; w.cfg = cfg; w.T = T; w.n_stride = n_stride; w.q = q; w.k_cache = k_cache;
    w.v_cache = v_cache; w.kv_lens = kv_lens; w.q_start = q_start; w.nrows = n; w.rows_b = ib;
    w.rows_i = ig; w.sel_in = sel; w.dout = dout; w.out = dq; w.dk = dk; w.dv = dv;
    const int rc = run_rows(&w, nthreads);
    free(ib);
    free(ig);
    return rc;
}

int oracle_index_pool_rows(const oracle_cfg *cfg, int32_t T, int64_t n_stride, const void *q_idx,
                           const void *k_idx, const int32_t *kv_lens, const int32_t *q_start,
                           int64_t nrows, const int32_t *rows_b, const int32_t *rows_i,
                           int32_t nthreads, int64_t nb_out, double *pooled) {
    row_work w = { 0 };
    w.kind = 3; w.cfg = cfg; w.T = T; w.n_stride = n_stride; w.q_idx = q_idx; w.k_idx = k_idx;
    w.kv_lens = kv_lens; w.q_start = q_start; w.nrows = nrows; w.rows_b = rows_b;
    w.rows_i = rows_i; w.nb_out = nb_out; w.pooled = pooled;
    return run_rows(&w, nthreads);
}

int oracle_sparse_attn_rows(const oracle_cfg *cfg, int32_t T, int64_t n_stride, const uint16_t *q,
                            const uint16_t *k_cache, const uint16_t *v_cache,
                            const int32_t *kv_lens, const int32_t *q_start, int64_t nrows,
                            const int32_t *rows_b, const int32_t *rows_i, const int32_t *sel_in,
                            int32_t nthreads, double *out, double *lse) {
    row_work w = { 0 };
    w.kind = 1; w.cfg = cfg; w.T = T; w.n_stride = n_stride; w.q = q; w.k_cache = k_cache;
    w.v_cache = v_cache; w.kv_lens = kv_lens; w.q_start = q_start; w.nrows = nrows;
    w.rows_b = rows_b; w.rows_i = rows_i; w.sel_in = sel_in; w.out = out; w.lse = lse;
    return run_rows(&w, nthreads);
}

int oracle_dense_causal_rows(const oracle_cfg *cfg, int32_t T, int64_t n_stride,
                             const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                             const int32_t *kv_lens, const int32_t *q_start, int64_t nrows,
                             const int32_t *rows_b, const int32_t *rows_i, int32_t nthreads,
                             double *out, double *lse) {
    row_work w = { 0 };
    w.kind = 2; w.cfg = cfg; w.T = T; w.n_stride = n_stride; w.q = q; w.k_cache = k_cache;
    w.v_cache = v_cache; w.kv_lens = kv_lens; w.q_start = q_start; w.nrows = nrows;
    w.rows_b = rows_b; w.rows_i = rows_i; w.out = out; w.lse = lse;
    return run_rows(&w, nthreads);
}

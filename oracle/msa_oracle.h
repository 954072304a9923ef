/*
 * CPU oracle for MiniMax Sparse Attention (MSA) — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 definition of what the method computes, used to check the
 * GPU library. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product path never calls it. It shares no
 * code, header, table or constant with the GPU library.
 *
 * Sources (web pages on MiniMax M3's sparse attention):
 *   [T]  cloud.tencent.com, "Something BIG Is Coming 百万token上下文提速近10倍，
 *        MiniMax M3的稀疏注意力凭什么这么快": §二 (index branch: one index
 *        query per GQA group, block max-pool, top-k; sparse branch: full
 *        attention over the chosen blocks), §六 (all heads of a GQA group
 *        share the chosen blocks).
 *   [M]  mlqm.cn, "如何用MiniMax-M3的稀疏注意力技术解决大模型效率瓶颈", section
 *        核心原理: sparse_attention_config (index dim 128, 4 index heads,
 *        top-k 16 blocks, block size 128).
 *
 * Parity status: every function here is pinned by the CPU tests (worked
 * example, brute force, dense-attention reduction, invariants).
 */
#ifndef MSA_ORACLE_H
#define MSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t groups;          /* G: KV heads = GQA groups = index heads            */
    int32_t heads_per_group; /* R: query heads per group; H = G*R                 */
    int32_t head_dim;        /* d                                                 */
    int32_t index_dim;       /* d_I                                               */
    int32_t block_size;      /* S: tokens per KV block                            */
    int32_t topk;            /* K: blocks kept per (query, group)                 */
    double softmax_scale;    /* tau; <= 0 selects 1/sqrt(d)                       */
    int32_t index_dtype;     /* 0: bfloat16, 1: FP8 E4M3FN (OCP)                  */
} oracle_cfg;

/* Element decoders (exact). */
double oracle_bf16_value(uint16_t bits);
double oracle_e4m3_value(uint8_t bits);

/*
 * Index scores and causal block max-pool for one query row at position p:
 * writes pooled[G * (p/S + 1)], pooled[g*(p/S+1) + beta] = max of the scores
 * of keys beta*S .. min(beta*S+S-1, p). Same argument layouts as below.
 */
int oracle_index_pool_row(const oracle_cfg *cfg, const void *q_idx_row, const void *k_idx_seq,
                          int64_t p, double *pooled);

/*
 * Index branch for one query row at position p (0 <= p < N):
 *   q_idx_row : [G, d_I] elements (bf16 or e4m3 per cfg->index_dtype)
 *   k_idx_seq : [N, d_I] elements of this sequence (row j = position j)
 * Writes sel[G*K] (block ids in (score desc, id asc) order, -1 padding) and,
 * if scores != NULL, scores[G*K] (pooled score of each chosen block, -inf pad).
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_index_topk_row(const oracle_cfg *cfg, const void *q_idx_row, const void *k_idx_seq,
                          int64_t p, int32_t *sel, double *scores);

/*
 * Query-block-shared selection (mlqm.cn article, section 核心原理: 128-token
 * blocks, each interacting with its 16 most relevant blocks), for query block
 * q_start / S + slot of one sequence: over the rows i of the call in that
 * block (position q_start + i < kv_len), a key block's score is the largest
 * of those rows' causal pooled scores; the top-K in (score desc, id asc)
 * order is shared by the block's rows. q_idx_seq [T, G, d_I]; k_idx_seq
 * [N, d_I]. Writes sel[G*K] and scores[G*K] (-1 / -inf when no row).
 */
int oracle_index_topk_qblock(const oracle_cfg *cfg, const void *q_idx_seq, int32_t T,
                             const void *k_idx_seq, int64_t q_start, int64_t kv_len,
                             int64_t slot, int32_t *sel, double *scores);

/*
 * Sparse branch for one query row at position p:
 *   q_row  : [H, d] bf16 bits
 *   k_seq, v_seq : [G, n_stride, d] bf16 bits (this sequence's caches)
 *   sel    : [G, K] block ids (any order; -1 entries ignored; repeats count once)
 * Writes out[H*d] and, if lse != NULL, lse[H] (natural log).
 */
int oracle_sparse_attn_row(const oracle_cfg *cfg, const uint16_t *q_row, const uint16_t *k_seq,
                           const uint16_t *v_seq, int64_t n_stride, int64_t p,
                           const int32_t *sel, double *out, double *lse);

/*
 * Backward of the sparse branch for fixed selections (the Tencent article's
 * §五 presents the design as trainable; the discrete selection carries no
 * gradient): for sequence data q_seq, dout_seq [T, H, d] (bf16 bits), one
 * group's caches k_grp, v_grp [n_stride, d], sel_seq [T, G, K], writes
 * dq_seq [T, H, d] for the heads of group g and dk_grp, dv_grp [n_stride, d]:
 *   P = softmax(tau q.k) over the row's kept keys, dP_j = dout.v_j,
 *   dS_j = P_j (dP_j - sum_k P_k dP_k), dq = tau sum dS_j k_j,
 *   dk_j += tau dS_j q, dv_j += P_j dout.
 */
int oracle_sparse_attn_backward_group(const oracle_cfg *cfg, int32_t T, int64_t n_stride,
                                      const uint16_t *q_seq, const uint16_t *k_grp,
                                      const uint16_t *v_grp, int64_t kv_len, int64_t q_start,
                                      int32_t g, const int32_t *sel_seq, const uint16_t *dout_seq,
                                      double *dq_seq, double *dk_grp, double *dv_grp);

/* Batched backward over every (sequence, group) on a thread pool: q, dout
 * [B, T, H, d], caches [B, G, n_stride, d], sel [B, T, G, K]; dq [B, T, H, d],
 * dk, dv [B, G, n_stride, d] (float64). */
int oracle_sparse_attn_backward(const oracle_cfg *cfg, int32_t B, int32_t T, int64_t n_stride,
                                const uint16_t *q, const uint16_t *k_cache,
                                const uint16_t *v_cache, const int32_t *kv_lens,
                                const int32_t *q_start, const int32_t *sel, const uint16_t *dout,
                                int32_t nthreads, double *dq, double *dk, double *dv);

/* Dense causal GQA softmax attention over every key j <= p (same layouts). */
int oracle_dense_causal_row(const oracle_cfg *cfg, const uint16_t *q_row, const uint16_t *k_seq,
                            const uint16_t *v_seq, int64_t n_stride, int64_t p,
                            double *out, double *lse);

/*
 * Many rows on a thread pool. Batched layouts (row-major, contiguous):
 *   q_idx [B, T, G, d_I], k_idx [B, n_stride, d_I], q [B, T, H, d],
 *   k_cache / v_cache [B, G, n_stride, d]; row r is (rows_b[r], rows_i[r]) and
 *   sits at position q_start[b] + i, which must be < kv_lens[b] <= n_stride.
 * Outputs are per listed row: sel [nrows, G, K], scores [nrows, G, K],
 * out [nrows, H, d], lse [nrows, H]. For the attention call, sel_in holds the
 * [nrows, G, K] block lists to attend over.
 */
int oracle_index_topk_rows(const oracle_cfg *cfg, int32_t T, int64_t n_stride, const void *q_idx,
                           const void *k_idx, const int32_t *kv_lens, const int32_t *q_start,
                           int64_t nrows, const int32_t *rows_b, const int32_t *rows_i,
                           int32_t nthreads, int32_t *sel, double *scores);

/* Query-block selections for items (items_b[r], items_slot[r]) with the
 * batched layouts above: sel / scores [nitems, G, K]. */
int oracle_index_topk_qblocks(const oracle_cfg *cfg, int32_t T, int64_t n_stride,
                              const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                              const int32_t *q_start, int64_t nitems, const int32_t *items_b,
                              const int32_t *items_slot, int32_t nthreads, int32_t *sel,
                              double *scores);

/* pooled [nrows, G, nb_out]: blocks past the row's position are -inf. */
int oracle_index_pool_rows(const oracle_cfg *cfg, int32_t T, int64_t n_stride, const void *q_idx,
                           const void *k_idx, const int32_t *kv_lens, const int32_t *q_start,
                           int64_t nrows, const int32_t *rows_b, const int32_t *rows_i,
                           int32_t nthreads, int64_t nb_out, double *pooled);

int oracle_sparse_attn_rows(const oracle_cfg *cfg, int32_t T, int64_t n_stride, const uint16_t *q,
                            const uint16_t *k_cache, const uint16_t *v_cache,
                            const int32_t *kv_lens, const int32_t *q_start, int64_t nrows,
                            const int32_t *rows_b, const int32_t *rows_i, const int32_t *sel_in,
                            int32_t nthreads, double *out, double *lse);

int oracle_dense_causal_rows(const oracle_cfg *cfg, int32_t T, int64_t n_stride,
                             const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                             const int32_t *kv_lens, const int32_t *q_start, int64_t nrows,
                             const int32_t *rows_b, const int32_t *rows_i, int32_t nthreads,
                             double *out, double *lse);

#ifdef __cplusplus
}
#endif
#endif

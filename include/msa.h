/*
 * msa.h — C ABI of libmsa, a gfx950 (MI355X) implementation of MiniMax Sparse
 * Attention (MSA).
 *
 * The method (web pages on MiniMax M3's sparse attention):
 *   - cloud.tencent.com, "Something BIG Is Coming 百万token上下文提速近10倍，
 *     MiniMax M3的稀疏注意力凭什么这么快", §二: an index branch in which one
 *     lightweight index query per GQA group scores the KV blocks, max-pools
 *     the scores over each block and keeps the top-k blocks; then a sparse
 *     branch that runs full attention over only the kept blocks. §六: all
 *     heads of one GQA group share the kept blocks.
 *   - mlqm.cn, "如何用MiniMax-M3的稀疏注意力技术解决大模型效率瓶颈", section
 *     核心原理: sparse_attention_config = index dim 128, 4 index heads,
 *     top-k 16 blocks, block size 128.
 *
 * Definitions used by every call. Sequence b, query row i sits at position
 * p = q_start[b] + i and may see keys j <= p (causal). For GQA group g:
 *   score  s_j  = sum_c q_idx[b,i,g,c] * k_idx[b,j,c]            (j <= p)
 *   pooled P_B  = max { s_j : B*S <= j <= min(B*S+S-1, p) }       (B*S <= p)
 *   sel[b,i,g,:] = the min(K, p/S+1) blocks of largest P_B, ordered by
 *                  (P_B descending, B ascending), then -1 padding.
 * For each query head h of group g (h in [g*R, (g+1)*R)), with
 *   J = { j <= p : j/S is in sel[b,i,g,:] } and tau = softmax scale:
 *   out[b,i,h,:] = sum_{j in J} softmax_j(tau * q[b,i,h,:].K[b,g,j,:]) V[b,g,j,:]
 *   lse[b,i,h]   = log sum_{j in J} exp(tau * q.K_j)   (natural log)
 * A row whose J is empty gets out = 0 and lse = -inf.
 *
 * Layouts (row-major, contiguous, device memory; bf16 = bfloat16 bits):
 *   q        [B, T, H, d]    bf16, H = G*R
 *   q_idx    [B, T, G, dI]   bf16 or FP8 E4M3FN (OCP) per cfg->index_dtype
 *   k_idx    [B, Nmax, dI]   same dtype as q_idx; one index key per token,
 *                            shared by all groups
 *   k_cache, v_cache [B, G, Nmax, d] bf16: each 128-token block of one group
 *                            is one contiguous 32 KiB run
 *   kv_lens  [B] int32       keys 0..kv_lens[b]-1 exist; kv_lens[b] <= Nmax
 *   q_start  [B] int32 or NULL (NULL: q_start[b] = kv_lens[b] - T)
 *   sel      [B, T, G, K] int32; sel_scores [B, T, G, K] fp32 (nullable)
 *   out      [B, T, H, d] bf16; lse [B, T, H] fp32 (nullable)
 *
 * Ownership and streams: the caller owns every buffer. The library allocates
 * nothing, keeps no state between calls and never synchronises: every call
 * enqueues its kernels on `stream` and returns. Scratch memory comes from the
 * caller's `workspace` (size from msa_workspace_size; a call whose size is 0,
 * such as msa_index_topk on a large prefill with K <= 32, accepts NULL): plain
 * scratch that needs no initialisation and may be reused by any later call on
 * the same stream. Calls that may run at the same time (other streams) must
 * not share a workspace.
 *
 * Errors: shapes, pointers, alignment (16 bytes for tensors, 4 for int32 and
 * fp32 arrays, 256 for the workspace) and workspace size are checked on the
 * host before any launch. Values that live on the device are not checked on
 * the host: a row whose position is outside [0, min(kv_lens[b], Nmax)) is
 * treated as empty (sel = -1, scores = -inf, out = 0, lse = -inf), and block
 * ids in `sel` outside the row's causal range are ignored, so no kernel reads
 * out of bounds. msa_last_error() describes the most recent failure on the
 * calling thread.
 *
 * Support limits: d = dI = S = 128; 1 <= K <= 64; 1 <= R <= 16; G >= 1;
 * B <= 65535 (the query-block variant: K <= 32). Results are deterministic
 * (no floating-point atomics).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MSA_OK = 0,
    MSA_ERR_INVALID_ARG = 1, /* null pointer, bad shape, misalignment      */
    MSA_ERR_UNSUPPORTED = 2, /* well-formed but outside the support limits */
    MSA_ERR_WORKSPACE = 3,   /* workspace missing or too small             */
    MSA_ERR_HIP = 4          /* a HIP launch or runtime call failed        */
} msa_status;

typedef enum { MSA_BF16 = 0, MSA_FP8_E4M3 = 1 } msa_dtype;

/* Which call a workspace is sized for. */
typedef enum {
    MSA_WS_INDEX_TOPK = 0,
    MSA_WS_SPARSE_PREFILL = 1,
    MSA_WS_SPARSE_DECODE = 2,
    MSA_WS_DECODE = 3,
    MSA_WS_SPARSE_BACKWARD = 4
} msa_ws_kind;

/* Layer shapes; the names follow the pages' sparse_attention_config. */
typedef struct {
    int32_t num_kv_groups;   /* G: KV heads = GQA groups = index heads        */
    int32_t heads_per_group; /* R: query heads per group                      */
    int32_t head_dim;        /* d (must be 128)                               */
    int32_t index_dim;       /* dI, sparse_index_dim (must be 128)            */
    int32_t block_size;      /* S, sparse_block_size (must be 128)            */
    int32_t topk;            /* K, sparse_topk_blocks (1..64)                 */
    float softmax_scale;     /* tau; 0 selects 1/sqrt(d)                      */
    int32_t index_dtype;     /* msa_dtype of q_idx and k_idx                  */
} msa_config;

/*
 * Index branch (Tencent article §二): scores, causal block max-pool and top-k
 * for B*T*G rows. Writes sel (and sel_scores if non-NULL: the pooled score of
 * each kept block, -inf for padding). T small enough that T*G <= 16 uses a
 * streaming kernel (decode); larger T uses an MFMA kernel (prefill), which
 * ranks each row's blocks in registers when K <= 32 and the call has at
 * least 64 tiles of 256 (row, group) rows (ceil(T*G/256) * B >= 64; no
 * workspace). Otherwise (K > 32, or a short prefill, whose key blocks are
 * then split over more workgroups) it writes the pooled scores to the
 * workspace and ranks them per row; msa_workspace_size gives
 * B*T*G*ceil(Nmax/S)*4 bytes (rounded up) then. Chunked prefill is
 * q_start[b] > 0 with the earlier keys already in k_idx.
 */
msa_status msa_index_topk(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                          const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                          const int32_t *q_start, int32_t *sel, float *sel_scores,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * First two steps of the index branch alone (Tencent article §二: index scores,
 * then the max over each block): pooled [B, T, G, nbm] fp32, nbm =
 * ceil(Nmax / S), with pooled[b,i,g,B'] = P_B' for every block B' <= p/S of a
 * row inside the cache. Other entries (blocks past the row's position, rows
 * outside the cache) are not written. Needs no workspace. Same dispatch as
 * msa_index_topk; the returned values are exact (integer-valued index data
 * give integer scores).
 */
msa_status msa_index_pool(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                          const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                          const int32_t *q_start, float *pooled, void *stream);

/*
 * Sparse branch for T query rows per sequence (Tencent article §二 and §六):
 * every head of group g attends over the blocks sel[b,i,g,:]. `sel` may come
 * from msa_index_topk or from the caller (repeated ids count once).
 */
msa_status msa_sparse_attn_prefill(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                   const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *kv_lens, const int32_t *q_start,
                                   const int32_t *sel, void *out, float *lse, void *workspace,
                                   size_t ws_bytes, void *stream);

/*
 * Sparse branch for one new token per sequence (T = 1, position kv_lens[b]-1;
 * the cache already holds that token): the kept blocks are split across
 * workgroups and merged by log-sum-exp. Same layouts with T = 1.
 */
msa_status msa_sparse_attn_decode(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                                  const void *k_cache, const void *v_cache,
                                  const int32_t *kv_lens, const int32_t *sel, void *out,
                                  float *lse, void *workspace, size_t ws_bytes, void *stream);

/*
 * One whole decode step of the method (index branch and sparse branch, Tencent
 * article §二 and §六): for every sequence b the new token at position
 * kv_lens[b]-1 (already in the caches) is scored against every cached index
 * key, its top-K blocks are written to sel (and sel_scores), and its G*R
 * heads attend over them into out (and lse). Equivalent to msa_index_topk
 * with T = 1 and q_start = NULL followed by msa_sparse_attn_decode, with one
 * workspace (MSA_WS_DECODE) for both. Same layouts with T = 1.
 */
msa_status msa_decode(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                      const void *q_idx, const void *k_idx, const void *k_cache,
                      const void *v_cache, const int32_t *kv_lens, int32_t *sel,
                      float *sel_scores, void *out, float *lse, void *workspace, size_t ws_bytes,
                      void *stream);

/*
 * msa_decode for callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * step and the same kernels, with its scratch memory (pooled block scores,
 * split partials, arrival counters) in a fixed array inside the library
 * instead of a caller workspace. The array holds
 * msa_decode_no_alloc_max_scratch() bytes (32 MiB) on every GPU the library
 * runs on, from that GPU's first call until the process ends; the first call
 * on a device looks up the array's address there. Shapes that need more
 * scratch than that (msa_workspace_size(cfg, B, 1, Nmax, MSA_WS_DECODE)) are
 * rejected with MSA_ERR_WORKSPACE before any launch. Arguments, outputs and
 * errors otherwise as msa_decode. Every call on one GPU shares that GPU's
 * array: calls that may overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller; a call's kernels reset the
 * state they need, so nothing carries over from the previous call.
 */
msa_status msa_decode_no_alloc(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                               const void *q_idx, const void *k_idx, const void *k_cache,
                               const void *v_cache, const int32_t *kv_lens, int32_t *sel,
                               float *sel_scores, void *out, float *lse, void *stream);

/* Bytes of the fixed scratch array msa_decode_no_alloc uses on each GPU. */
size_t msa_decode_no_alloc_max_scratch(void);

/*
 * Backward of the sparse branch for fixed selections (the Tencent article's
 * §五 presents the two-branch design as trainable; the discrete selection
 * carries no gradient). With J, P and tau as in the forward definition,
 * dout the gradient of out, dP_j = dout.v_j and dS_j = P_j (dP_j - sum_k
 * P_k dP_k):
 *   dq[b,i,h,:] = tau sum_j dS_j K[b,g,j,:]
 *   dk[b,g,j,:] = tau sum over (row, head of g) attending j of dS_j q
 *   dv[b,g,j,:] = sum over (row, head of g) attending j of P_j dout
 * Inputs: the forward's q, caches, kv_lens, q_start, sel, out (bf16) and lse
 * (fp32, natural log, as msa_sparse_attn_prefill writes them), dout [B,T,H,d]
 * bf16. Outputs, fp32 and overwritten whole: dq [B,T,H,d] (zero for rows
 * outside the cache), dk, dv [B,G,Nmax,d] (zero where no row attends).
 * Workspace MSA_WS_SPARSE_BACKWARD.
 */
msa_status msa_sparse_attn_backward(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                    const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *kv_lens, const int32_t *q_start,
                                    const int32_t *sel, const void *out, const float *lse,
                                    const void *dout, float *dq, float *dk, float *dv,
                                    void *workspace, size_t ws_bytes, void *stream);

/*
 * Query-block-shared selection, a variant of the index branch read from the
 * mlqm.cn article, section 核心原理 (the sequence is cut into 128-token blocks
 * and each block works with its 16 most relevant blocks). The query block of
 * the row at position p is p / S, the same blocks as the keys. For each
 * sequence, group and query block, over the rows of the call in that block
 * (positions below kv_lens[b]), a key block's score is the largest pooled
 * score P_B that any of those rows gives it (each row pooling causally, as
 * above), and the top-K in (score desc, block asc) order, then -1 padding,
 * is shared by every row of the query block.
 *   sel        [B, NQ, G, K] int32, NQ = msa_qblock_slots(T); slot s holds
 *              query block floor(q_start[b] / S) + s (a slot with no row of
 *              the call gets -1);
 *   sel_scores [B, NQ, G, K] fp32 (nullable), -inf for padding.
 * Other layouts as msa_index_topk. Needs no workspace. Exact for integer
 * index data, as msa_index_topk. K <= 32 (the ranking is kept in registers);
 * larger K returns MSA_ERR_UNSUPPORTED.
 */
msa_status msa_index_topk_qblock(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                 const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                                 const int32_t *q_start, int32_t *sel, float *sel_scores,
                                 void *stream);

/*
 * Sparse branch for query-block-shared selections: row i of sequence b
 * (position p = q_start[b] + i) attends, for every head of group g, over the
 * keys j <= p of the blocks in sel[b, p/S - floor(q_start[b]/S), g, :]
 * (invalid or repeated ids are ignored, as in msa_sparse_attn_prefill).
 * sel as written by msa_index_topk_qblock; other layouts and the output
 * definition as msa_sparse_attn_prefill. Needs no workspace: every query
 * block's rows attend over its kept blocks in one pass (online softmax).
 */
msa_status msa_sparse_attn_prefill_qblock(const msa_config *cfg, int32_t B, int32_t T,
                                          int32_t Nmax, const void *q, const void *k_cache,
                                          const void *v_cache, const int32_t *kv_lens,
                                          const int32_t *q_start, const int32_t *sel, void *out,
                                          float *lse, void *stream);

/* Query-block slots NQ of a call with T rows per sequence: the number of
 * 128-token blocks that T consecutive positions can touch, ceil((T-1)/128)+1
 * (0 for T <= 0). */
int32_t msa_qblock_slots(int32_t T);

/*
 * Appends T new tokens per sequence to the caches that the calls above read
 * (the decode step's reading of the Tencent article §二 is that the new
 * token's K, V and index key are in the caches when it attends): for every
 * sequence b, row t < T and group g, with pos = pos0[b] + t,
 *   k_cache[b,g,pos,:] = k_new[b,t,g,:]    v_cache[b,g,pos,:] = v_new[b,t,g,:]
 *   k_idx[b,pos,:]     = k_idx_new[b,t,:]
 * Rows with pos outside [0, Nmax) are skipped (pos0 lives on the device and is
 * not checked on the host). Layouts: k_new, v_new [B, T, G, d] bf16;
 * k_idx_new [B, T, dI] in cfg->index_dtype; pos0 [B] int32. The bytes are
 * copied unchanged. Needs no workspace. A caller that appends at the old
 * length then passes kv_lens = old length + T to the calls above.
 */
msa_status msa_cache_append(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                            const void *k_new, const void *v_new, const void *k_idx_new,
                            const int32_t *pos0, void *k_cache, void *v_cache, void *k_idx,
                            void *stream);

/*
 * Index projections, the step ahead of the index branch: the Tencent
 * article (§二) forms one lightweight index query per GQA group from each
 * token's hidden state (n' x h x d -> n' x 1 x d), and the index keys it
 * scores against come from the tokens in the same way. The pages give no
 * weights, hidden size or quantisation; this call is the plain linear map:
 * for M token rows,
 *   q_idx[m, g, c] = sum_k hidden[m, k] * w[g*dI + c, k]      (g < G)
 *   k_idx[m, c]    = sum_k hidden[m, k] * w[G*dI + c, k]
 * accumulated in fp32 and rounded to bf16 (nearest even).
 * Layouts: hidden [M, hidden_dim] bf16; w [(G+1)*dI, hidden_dim] bf16 (the G
 * index-query projections, then the index-key projection, one output feature
 * per row); q_idx [M, G, dI] bf16 (for B sequences of T rows: [B, T, G, dI],
 * the layout msa_index_topk reads); k_idx [M, dI] bf16, nullable (then only
 * the queries are computed; msa_cache_append places new keys in the cache).
 * hidden_dim must be a multiple of 64; cfg->index_dtype must be MSA_BF16
 * (E4M3 index data need a quantisation the pages do not define:
 * MSA_ERR_UNSUPPORTED). Needs no workspace.
 */
msa_status msa_index_project(const msa_config *cfg, int32_t M, int32_t hidden_dim,
                             const void *hidden, const void *w, void *q_idx, void *k_idx,
                             void *stream);

/* Workspace bytes the named call needs for these shapes (0 if none); returns
 * (size_t)-1 for an invalid configuration. For MSA_WS_SPARSE_DECODE and
 * MSA_WS_DECODE, T is 1. */
size_t msa_workspace_size(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                          int32_t which);

const char *msa_status_string(msa_status s);
const char *msa_last_error(void);
/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t msa_version(void);

#ifdef __cplusplus
}
#endif
#endif

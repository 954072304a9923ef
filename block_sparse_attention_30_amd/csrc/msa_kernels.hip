// libmsa kernels for gfx950 (MI355X, CDNA4) and the C-ABI entry points that
// launch them.
//
// The method (MiniMax M3 sparse attention, cloud.tencent.com article
// "Something BIG Is Coming 百万token上下文提速近10倍，MiniMax M3的稀疏注意力凭什么这么快"):
//   §二 index branch: one index query per GQA group scores the KV blocks
//       (block max-pool of per-token scores) and keeps the top-k blocks;
//   §二 sparse branch: full softmax attention over only the kept blocks;
//   §六 all heads of a GQA group share the kept blocks, which are loaded once.
// Sizes (block 128, top-k 16, index dim 128) are the sparse_attention_config
// of the mlqm.cn guide "如何用MiniMax-M3的稀疏注意力技术解决大模型效率瓶颈", §核心原理.
//
// Kernels:
//   idx_scan_kernel     decode index scores: streams k_idx once for all groups,
//                       16x16x32 bf16 MFMA, causal block max in registers.
//   idx_prefill_kernel  prefill index scores: 32x32x16 bf16 MFMA over a 256-row
//                       tile with the k_idx block staged in LDS; block max-pool
//                       in the epilogue.
//   topk_kernel         one wavefront per row: bitonic sort of 64-bit keys
//                       (score, inverted block id) across lanes plus ballot
//                       compaction of candidates above the running threshold.
//   sparse_attn_kernel  gathers the kept 128-token K/V blocks of one group,
//                       serves all R heads of the group with 16x16x32 MFMA
//                       (QK^T and PV) and an online fp32 softmax.
//   combine_kernel      log-sum-exp merge of split partials (decode).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "msa_internal.h"

namespace {

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int S = msa::kBlock;
constexpr int D = msa::kHeadDim;
constexpr int DI = msa::kIndexDim;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t *p) { return as_bf16x8(ld16(p)); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    u32x4 z = {0u, 0u, 0u, 0u};
    return as_bf16x8(z);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_kv(int kv, int Nmax) { return kv < Nmax ? kv : Nmax; }

// ---------------------------------------------------------------------------
// Decode index scores (T*G <= 16 rows per sequence).
//
// MFMA D = A x B with A = index-query rows (16 rows: m = t*G + g, zero above
// T*G) and B = k_idx^T for 16 tokens. Lane l loads 16 contiguous bytes of
// token (l & 15) per k-chunk, so each wave reads 4 KiB of k_idx per tile.
// Output lane l holds D[4*(l>>4) + r][l & 15]: rows 4*(l>>4)..+3 of one token.
// A running max per row over the block's 8 tiles, then a 16-lane max,
// gives the pooled score of the block.
__global__ __launch_bounds__(256) void idx_scan_kernel(
    const bf16_t *__restrict__ q_idx, const bf16_t *__restrict__ k_idx,
    const int32_t *__restrict__ kv_lens, const int32_t *__restrict__ q_start,
    float *__restrict__ pooled, int T, int G, int Nmax, int64_t nb_max, int blocks_per_wg) {
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rows = T * G;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int p_hi = min(qs + T - 1, kv - 1);
    if (p_hi < 0) return;
    const int nb = p_hi / S + 1;
    const int blk_begin = blockIdx.x * blocks_per_wg;
    if (blk_begin >= nb) return;
    const int blk_end = min(blk_begin + blocks_per_wg, nb);

    const int col = lane & 15, kg = lane >> 4;
    bf16x8 a[4];
    {
        const bf16_t *qp = q_idx + ((size_t)b * rows + (col < rows ? col : 0)) * DI + kg * 8;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) a[kc] = col < rows ? ld_bf16x8(qp + kc * 32) : zero_bf16x8();
    }
    int prow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kg + r;
        const int p = qs + m / G;
        prow[r] = (m < rows && p >= 0 && p < kv) ? p : -1;
    }
    const bf16_t *kseq = k_idx + (size_t)b * Nmax * DI + kg * 8;
    for (int blk = blk_begin + wave; blk < blk_end; blk += 4) {
        const int tok0 = blk * S;
        const bool need_mask = tok0 + S - 1 > qs;
        float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int tile = 0; tile < S / 16; ++tile) {
            const int tok = tok0 + tile * 16 + col;
            const int tok_ld = tok < kv ? tok : kv - 1;  // stay inside the cache
            const bf16_t *kp = kseq + (size_t)tok_ld * DI;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) acc = mfma16(a[kc], ld_bf16x8(kp + kc * 32), acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float s = (need_mask && tok > prow[r]) ? -INFINITY : acc[r];
                mx[r] = fmaxf(mx[r], s);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mx[r] = fmaxf(mx[r], __shfl_xor(mx[r], off));
        }
        if (col == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (prow[r] >= tok0)
                    pooled[((size_t)b * rows + 4 * kg + r) * nb_max + blk] = mx[r] + 0.0f;
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill index scores. A workgroup owns 256 consecutive (query, group) rows
// of one sequence; wave w owns rows [64w, 64w+64) as two 32-column MFMA tiles
// whose index queries stay in registers (B operand). For each causal KV block
// the 128 x 128 k_idx tile is staged once in LDS (rows padded to 272 bytes so
// that 16 lanes reading 16 bytes each hit distinct banks) and read as the A
// operand by all four waves. D lane l holds column (l & 31) and rows
// 8*(i>>2) + 4*(l>>5) + (i&3), so the block max of a column is an in-lane max
// over the four row tiles plus one exchange with lane l^32.
constexpr int kPfRows = 256;
constexpr int kLdsRow = 272;

__global__ __launch_bounds__(256) void idx_prefill_kernel(
    const bf16_t *__restrict__ q_idx, const bf16_t *__restrict__ k_idx,
    const int32_t *__restrict__ kv_lens, const int32_t *__restrict__ q_start,
    float *__restrict__ pooled, int T, int G, int Nmax, int64_t nb_max) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[S * kLdsRow];
    const int b = blockIdx.y;
    const int rows = T * G;
    const int r0 = (gridDim.x - 1 - blockIdx.x) * kPfRows;  // longest rows first
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int r_last = min(r0 + kPfRows, rows) - 1;
    const int p_hi = min(qs + r_last / G, kv - 1);
    if (p_hi < 0) return;
    const int p_lo = qs + r0 / G;
    const int nblk = p_hi / S + 1;

    const int j = lane & 31, half = lane >> 5;
    bf16x8 qb[2][8];
    int pcol[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int r = r0 + 64 * wave + 32 * ct + j;
        const int p = qs + r / G;
        const bool ok = r < rows && p >= 0 && p < kv;
        pcol[ct] = ok ? p : -1;
        const bf16_t *qp = q_idx + ((size_t)b * rows + (ok ? r : 0)) * DI + half * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qb[ct][ks] = ok ? ld_bf16x8(qp + ks * 16) : zero_bf16x8();
    }
    const bf16_t *kseq = k_idx + (size_t)b * Nmax * DI;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    for (int blk = 0; blk < nblk; ++blk) {
        const int tok0 = blk * S;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int piece = tid + 256 * i;
            const int tk = piece >> 4, c = piece & 15;
            const int tok = tok0 + tk;
            const u32x4 v = tok < kv ? ld16(kseq + (size_t)tok * DI + c * 8) : zero4;
            *reinterpret_cast<u32x4 *>(lds + tk * kLdsRow + c * 16) = v;
        }
        __syncthreads();
        const bool need_mask = tok0 + S - 1 > p_lo;
        float cm0 = -INFINITY, cm1 = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x16 acc0 = {}, acc1 = {};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 a = as_bf16x8(
                    *reinterpret_cast<const u32x4 *>(lds + (rt * 32 + j) * kLdsRow + ks * 32 + half * 16));
                acc0 = mfma32(a, qb[0][ks], acc0);
                acc1 = mfma32(a, qb[1][ks], acc1);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tok = tok0 + rt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                float s0 = acc0[i], s1 = acc1[i];
                if (need_mask) {
                    if (tok > pcol[0]) s0 = -INFINITY;
                    if (tok > pcol[1]) s1 = -INFINITY;
                }
                cm0 = fmaxf(cm0, s0);
                cm1 = fmaxf(cm1, s1);
            }
        }
        cm0 = fmaxf(cm0, __shfl_xor(cm0, 32));
        cm1 = fmaxf(cm1, __shfl_xor(cm1, 32));
        const float v = half ? cm1 : cm0;
        const int pc = half ? pcol[1] : pcol[0];
        const int r = r0 + 64 * wave + 32 * half + j;
        if (pc >= tok0) pooled[((size_t)b * rows + r) * nb_max + blk] = v + 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Top-k over the pooled scores of one row. Keys are unique 64-bit integers:
// the fp32 score mapped to an order-preserving uint32 (negative zero taken as
// zero) in the high half and 0xFFFFFFFF - block in the low half, so a larger
// key is a better block and equal scores rank the lower block first. Key 0 is
// "no block".
__device__ __forceinline__ uint64_t score_key(float s, int blk) {
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)blk);
}

__device__ __forceinline__ float key_score(uint64_t k) {
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ int key_block(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    const int lo = __shfl((int)(uint32_t)v, src), hi = __shfl((int)(uint32_t)(v >> 32), src);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const int lo = __shfl_xor((int)(uint32_t)v, m), hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Bitonic sort of one key per lane across the 64-lane wavefront, descending
// (lane 0 ends with the largest key).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x, int lane) {
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t y = shfl_xor_u64(x, j);
            const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
            x = keep_max ? (x > y ? x : y) : (x < y ? x : y);
        }
    }
    return x;
}

// Position of the r-th (0-based) set bit of mask, or -1.
__device__ __forceinline__ int nth_set_bit(uint64_t mask, int r) {
    if (r < 0 || r >= __popcll(mask)) return -1;
    int pos = 0;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const uint64_t low = (pos + s >= 64) ? ~0ull : ((1ull << (pos + s)) - 1ull);
        if (__popcll(mask & low) <= r) pos += s;
    }
    return pos;
}

// One wavefront per row (b, t, g). Pass 1: every lane takes the best key of
// its strided share; the K best of those 64 are a valid running top-K and the
// K-th is a threshold below which no key can enter. Pass 2 walks the row in
// rounds of 64 keys; keys above the threshold (rare after pass 1) are
// compacted into lanes K..63 next to the current top-K and the 64 are sorted.
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ pooled, int64_t nb_max, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, int B, int T, int G, int Nmax, int K,
    int32_t *__restrict__ sel, float *__restrict__ sel_scores) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int rows = T * G;
    if (row >= (int64_t)B * rows) return;
    const int b = (int)(row / rows);
    const int t = (int)(row % rows) / G;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int p = qs + t;
    int32_t *out = sel + row * K;
    float *outs = sel_scores ? sel_scores + row * K : nullptr;
    if (p < 0 || p >= kv) {
        if (lane < K) {
            out[lane] = -1;
            if (outs) outs[lane] = -INFINITY;
        }
        return;
    }
    const int n = p / S + 1;
    const float *cand = pooled + row * nb_max;
    uint64_t lmax = 0;
    for (int i = lane; i < n; i += 64) {
        const uint64_t k = score_key(cand[i], i);
        lmax = k > lmax ? k : lmax;
    }
    uint64_t srt = wave_sort_desc(lmax, lane);
    uint64_t top = lane < K ? srt : 0;
    uint64_t thr = shfl_u64(srt, K - 1);
    const uint64_t below = (1ull << lane) - 1ull;
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        const uint64_t kk = i < n ? score_key(cand[i], i) : 0;
        bool q = kk > thr && kk != lmax;
        uint64_t qm = __ballot(q);
        while (qm) {
            const int rank = __popcll(qm & below);
            const bool take = q && rank < 64 - K;
            const uint64_t tm = __ballot(take);
            const int src = nth_set_bit(tm, lane - K);
            const uint64_t got = shfl_u64(kk, src < 0 ? 0 : src);
            uint64_t x = lane < K ? top : (src >= 0 ? got : 0);
            x = wave_sort_desc(x, lane);
            top = lane < K ? x : 0;
            thr = shfl_u64(x, K - 1);
            q = q && !take && kk > thr;
            qm = __ballot(q);
        }
    }
    if (lane < K) {
        out[lane] = top ? key_block(top) : -1;
        if (outs) outs[lane] = top ? key_score(top) : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Block-sparse attention. One workgroup (4 waves) per (sequence, row, group,
// split); split s covers kept slots [s*spl, s*spl + spl). Every kept block is
// cut into four 32-token chunks and wave w takes chunk w of each block, so a
// block is read once per workgroup and its K/V serve all R heads of the group.
//
// Per chunk (16x16x32 bf16 MFMA):
//   S^T = K x q^T : A = 16 tokens of K (16 contiguous bytes per lane straight
//                   from the cache), B = the group's query heads (zero above R).
//                   Lane l holds heads (l & 15), tokens 4*(l>>4)+r.
//   online softmax in the log2 domain, fp32;
//   O  += P x V   : A = P, taken from the lane's own S^T values (two 16-token
//                   tiles give 8 tokens), B = V read from an LDS copy of the
//                   chunk stored transposed ([d][token]).
// The four waves' (m, l, O) are merged in LDS; with one split the row's output
// is written directly, otherwise an unnormalised partial and (m, l).
constexpr int kVtStride = 36;  // bf16 per transposed V row: 32 tokens + pad (72 bytes)

__global__ __launch_bounds__(256) void sparse_attn_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache,
    const bf16_t *__restrict__ v_cache, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const int32_t *__restrict__ sel, int T, int G, int R,
    int Nmax, int K, int spl, int nsplit, float scale_log2, bf16_t *__restrict__ out,
    float *__restrict__ lse, float *__restrict__ part_o, float *__restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[4 * D * kVtStride * 2];
    __shared__ int s_blocks[msa::kMaxTopk];
    __shared__ int s_nblk;
    __shared__ float s_m[4][16], s_l[4][16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t item = blockIdx.x;
    const int split = (int)(item % nsplit);
    const int g = (int)((item / nsplit) % G);
    const int64_t bt = item / ((int64_t)nsplit * G);
    const int b = (int)(bt / T), t = (int)(bt % T);
    const int H = G * R;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int p = qs + t;
    const bool row_ok = p >= 0 && p < kv;

    if (tid == 0) {
        int n = 0;
        if (row_ok) {
            const int32_t *srow = sel + (bt * G + g) * K;
            const int n_valid = p / S + 1;
            const int k_end = min(K, split * spl + spl);
            for (int k = split * spl; k < k_end; ++k) {
                const int blk = srow[k];
                if (blk < 0 || blk >= n_valid) continue;
                bool dup = false;
                for (int k2 = 0; k2 < k; ++k2) dup |= srow[k2] == blk;
                if (!dup) s_blocks[n++] = blk;
            }
        }
        s_nblk = n;
    }
    __syncthreads();
    const int nblk = s_nblk;

    const int col = lane & 15, kg = lane >> 4;
    bf16x8 qf[4];
    {
        const bool hv = col < R;
        const bf16_t *qp = q + (bt * H + g * R + (hv ? col : 0)) * D + kg * 8;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) qf[kc] = hv ? ld_bf16x8(qp + kc * 32) : zero_bf16x8();
    }
    const bf16_t *kg_base = k_cache + ((size_t)b * G + g) * Nmax * D;
    const bf16_t *vg_base = v_cache + ((size_t)b * G + g) * Nmax * D;
    bf16_t *vt = reinterpret_cast<bf16_t *>(smem) + wave * D * kVtStride;

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < nblk; ++c) {
        const int tok0 = s_blocks[c] * S + wave * 32;
        // S^T for two 16-token tiles.
        f32x4 st[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int tok = tok0 + rt * 16 + col;
            const int tok_ld = tok <= p ? tok : p;
            const bf16_t *kp = kg_base + (size_t)tok_ld * D + kg * 8;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) acc = mfma16(ld_bf16x8(kp + kc * 32), qf[kc], acc);
            st[rt] = acc;
        }
        // Transposed V chunk into this wave's LDS region; tokens past p are zero.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int piece = lane + 64 * i;
            const int tk = piece >> 4, cc = piece & 15;
            const int tok = tok0 + tk;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (tok <= p) v = ld16(vg_base + (size_t)tok * D + cc * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt[(cc * 8 + 2 * e) * kVtStride + tk] = (bf16_t)(v[e] & 0xFFFFu);
                vt[(cc * 8 + 2 * e + 1) * kVtStride + tk] = (bf16_t)(v[e] >> 16);
            }
        }
        // Online softmax (log2 domain). Lane holds head `col`, tokens
        // 4*kg + r (tile 0) and 16 + 4*kg + r (tile 1).
        float z[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = tok0 + rt * 16 + 4 * kg + r;
                z[rt][r] = tok <= p ? st[rt][r] * scale_log2 : -INFINITY;
                mx = fmaxf(mx, z[rt][r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
        float psum = 0.f;
        bf16x8 pa;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pv = m_new == -INFINITY ? 0.f : exp2f(z[rt][r] - m_new);
                psum += pv;
                pa[rt * 4 + r] = (__bf16)pv;
            }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        float a_row[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a_row[r] = __shfl(alpha, 4 * kg + r);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const bf16_t *vr = vt + (dt * 16 + col) * kVtStride + 4 * kg;
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr);
            const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 16);
            const u32x4 vb = {lo[0], lo[1], hi[0], hi[1]};
            f32x4 acc = o[dt];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= a_row[r];
            o[dt] = mfma16(pa, as_bf16x8(vb), acc);
        }
    }

    // Merge the four waves.
    if (lane < 16) {
        s_m[wave][lane] = m_run;
        s_l[wave][lane] = l_run;
    }
    __syncthreads();
    float *s_o = reinterpret_cast<float *>(smem);  // [4][16][128] fp32, reuses the V area
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * kg + r;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
        const float mw = s_m[wave][h];
        const float sc = mw == -INFINITY ? 0.f : exp2f(mw - M);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) s_o[(wave * 16 + h) * D + dt * 16 + col] = o[dt][r] * sc;
    }
    __syncthreads();
    const int64_t unit = bt * G + g;  // (row, group)
    for (int idx = tid; idx < R * D; idx += 256) {
        const int h = idx / D, dd = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (s_m[w][h] != -INFINITY) L += exp2f(s_m[w][h] - M) * s_l[w][h];
            acc += s_o[(w * 16 + h) * D + dd];
        }
        if (nsplit == 1) {
            const float val = L > 0.f ? acc / L : 0.f;
            __bf16 hv = (__bf16)val;
            out[(bt * H + g * R + h) * D + dd] = __builtin_bit_cast(bf16_t, hv);
            if (lse && dd == 0) lse[bt * H + g * R + h] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
        } else {
            const int64_t pu = (unit * nsplit + split) * R + h;
            part_o[pu * D + dd] = acc;
            if (dd == 0) {
                part_ml[pu * 2] = M;
                part_ml[pu * 2 + 1] = L;
            }
        }
    }
}

// Log-sum-exp merge of the nsplit partials of one (row, group).
__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_ml, int G, int R,
    int nsplit, bf16_t *__restrict__ out, float *__restrict__ lse) {
    const int64_t unit = blockIdx.x;  // (row, group)
    const int g = (int)(unit % G);
    const int64_t bt = unit / G;
    const int H = G * R;
    for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x) {
        const int h = idx / D, dd = idx % D;
        float M = -INFINITY;
        for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((unit * nsplit + s) * R + h) * 2]);
        float L = 0.f, acc = 0.f;
        if (M != -INFINITY) {
            for (int s = 0; s < nsplit; ++s) {
                const int64_t pu = (unit * nsplit + s) * R + h;
                const float ms = part_ml[pu * 2];
                if (ms == -INFINITY) continue;
                const float w = exp2f(ms - M);
                L += w * part_ml[pu * 2 + 1];
                acc += w * part_o[pu * D + dd];
            }
        }
        const float val = L > 0.f ? acc / L : 0.f;
        __bf16 hv = (__bf16)val;
        out[(bt * H + g * R + h) * D + dd] = __builtin_bit_cast(bf16_t, hv);
        if (lse && dd == 0) lse[bt * H + g * R + h] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
    }
}

msa_status launch_status(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return msa::fail(MSA_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
    return MSA_OK;
}

float scale_log2_of(const msa_config *cfg) {
    const float tau = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / sqrtf((float)cfg->head_dim);
    return tau * kLog2e;
}

}  // namespace

extern "C" {

msa_status msa_index_topk(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                          const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                          const int32_t *q_start, int32_t *sel, float *sel_scores,
                          void *workspace, size_t ws_bytes, void *stream) {
    msa::clear_error();
    msa_status s = msa::check_index_args(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, sel,
                                         sel_scores, workspace, ws_bytes);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    if (cfg->index_dtype != MSA_BF16)
        return msa::fail(MSA_ERR_UNSUPPORTED, "FP8 index keys are not supported by this build");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const msa::IndexWs w = msa::index_ws(cfg, B, T, Nmax);
    float *pooled = reinterpret_cast<float *>(static_cast<char *>(workspace) + w.pooled_off);
    const int G = cfg->num_kv_groups;
    const int rows = T * G;
    const bf16_t *qi = static_cast<const bf16_t *>(q_idx);
    const bf16_t *ki = static_cast<const bf16_t *>(k_idx);
    if (rows <= msa::kScanMaxRows) {
        int64_t per_wg = ((int64_t)B * w.nb_max + 2047) / 2048;
        per_wg = per_wg < 4 ? 4 : (per_wg + 3) / 4 * 4;
        const dim3 grid((unsigned)((w.nb_max + per_wg - 1) / per_wg), (unsigned)B);
        idx_scan_kernel<<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G, Nmax,
                                              w.nb_max, (int)per_wg);
    } else {
        const dim3 grid((unsigned)((rows + kPfRows - 1) / kPfRows), (unsigned)B);
        idx_prefill_kernel<<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G, Nmax,
                                                 w.nb_max);
    }
    if ((s = launch_status("index scoring kernel")) != MSA_OK) return s;
    const int64_t nrows = (int64_t)B * rows;
    topk_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(pooled, w.nb_max, kv_lens, q_start,
                                                            B, T, G, Nmax, cfg->topk, sel,
                                                            sel_scores);
    return launch_status("top-k kernel");
}

static msa_status sparse_call(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                              const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *kv_lens, const int32_t *q_start, const int32_t *sel,
                              void *out, float *lse, void *workspace, size_t ws_bytes,
                              void *stream, int32_t which) {
    msa::clear_error();
    msa_status s = msa::check_sparse_args(cfg, B, T, Nmax, q, k_cache, v_cache, kv_lens, q_start,
                                          sel, out, lse, workspace, ws_bytes, which);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const msa::SparseWs w = msa::sparse_ws(cfg, B, T, Nmax, which);
    const int G = cfg->num_kv_groups, R = cfg->heads_per_group, K = cfg->topk;
    const int nsplit = w.nsplit;
    const int spl = (K + nsplit - 1) / nsplit;
    float *part_o = nullptr, *part_ml = nullptr;
    if (nsplit > 1) {
        part_o = reinterpret_cast<float *>(static_cast<char *>(workspace) + w.part_o_off);
        part_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + w.part_ml_off);
    }
    const int64_t items = (int64_t)B * T * G * nsplit;
    sparse_attn_kernel<<<(unsigned)items, 256, 0, st>>>(
        static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k_cache),
        static_cast<const bf16_t *>(v_cache), kv_lens, q_start, sel, T, G, R, Nmax, K, spl,
        nsplit, scale_log2_of(cfg), static_cast<bf16_t *>(out), lse, part_o, part_ml);
    if ((s = launch_status("sparse attention kernel")) != MSA_OK) return s;
    if (nsplit > 1) {
        combine_kernel<<<(unsigned)((int64_t)B * T * G), 256, 0, st>>>(
            part_o, part_ml, G, R, nsplit, static_cast<bf16_t *>(out), lse);
        if ((s = launch_status("combine kernel")) != MSA_OK) return s;
    }
    return MSA_OK;
}

msa_status msa_sparse_attn_prefill(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                   const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *kv_lens, const int32_t *q_start,
                                   const int32_t *sel, void *out, float *lse, void *workspace,
                                   size_t ws_bytes, void *stream) {
    return sparse_call(cfg, B, T, Nmax, q, k_cache, v_cache, kv_lens, q_start, sel, out, lse,
                       workspace, ws_bytes, stream, MSA_WS_SPARSE_PREFILL);
}

msa_status msa_sparse_attn_decode(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                                  const void *k_cache, const void *v_cache,
                                  const int32_t *kv_lens, const int32_t *sel, void *out,
                                  float *lse, void *workspace, size_t ws_bytes, void *stream) {
    return sparse_call(cfg, B, 1, Nmax, q, k_cache, v_cache, kv_lens, nullptr, sel, out, lse,
                       workspace, ws_bytes, stream, MSA_WS_SPARSE_DECODE);
}

}  // extern "C"

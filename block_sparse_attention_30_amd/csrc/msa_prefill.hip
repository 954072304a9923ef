// libmsa prefill kernels for gfx950 (MI355X, CDNA4) and the prefill entry points.
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
//   idx_prefill_kernel   prefill index scores: 32x32x16 bf16 (or 32x32x64
//                        E4M3) MFMA over a 256-row tile with the k_idx block
//                        staged in LDS; block max-pool and a per-row running
//                        top-K in registers in the epilogue, or (pooled
//                        scores only: K above the register top-K, short
//                        prefills) the block maxima written out, with a short
//                        prefill's key blocks split over more workgroups.
//   sparse_attn_kernel   (small prefill) one workgroup per (row, group):
//                        gathers the kept 128-token K/V blocks, serves all R
//                        heads of the group with 16x16x32 MFMA (QK^T and PV)
//                        and an online fp32 softmax.
//   pf_*_kernel          (prefill) KV-major sparse attention: per-block entry
//                        lists, one staged block per workgroup serving every
//                        (row, head) that kept it, log-sum-exp merge.
//   pf_clear_kernel      zeroes the list bitmaps (a kernel, not a memset, so
//                        the calls can be captured in graphs).
//   cache_append_kernel  (msa_cache_append) copies new K, V and index-key rows
//                        into the caches, one wavefront per (sequence, row).
//   idx_prefill_kernel<.., QB> and qb_attn_kernel  the query-block-shared
//                        selection variant (msa_index_topk_qblock,
//                        msa_sparse_attn_prefill_qblock): one top-K per
//                        128-row query block; attention query-major with an
//                        online softmax over the block's kept blocks.
#include <algorithm>
#include "msa_device.h"

namespace {

// ---------------------------------------------------------------------------
// Prefill index scores. A workgroup owns 256 consecutive (query, group) rows
// of one sequence; wave w owns rows [64w, 64w+64) as two 32-column MFMA tiles
// whose index queries stay in registers (B operand). For each causal KV block
// the 128-token k_idx tile is staged once in LDS by direct global->LDS loads
// into one of two buffers (the next block streams in while this one is used;
// one barrier per block) and read as the A operand by all four waves. Rows are
// unpadded; the 16-byte pieces of a row are XOR-swizzled (idx_swz) so that 16
// lanes reading the same piece of 16 rows hit distinct banks. D lane l holds column (l & 31) and rows
// 8*(i>>2) + 4*(l>>5) + (i&3), so the block max of a column is an in-lane max
// over the four row tiles plus one exchange with lane l^32. bf16 keys use
// 32x32x16 bf16 MFMAs (8 per row tile and column tile), OCP E4M3 keys
// 32x32x64 f8f6f4 MFMAs with unit scales (2 per row tile and column tile).
constexpr int kPfRows = msa::kIdxTileRows;

// Physical 16-byte slot of logical piece `piece` of k_idx row `row` in the
// staged tile: bf16 rows (16 pieces) swizzle by row & 15; E4M3 rows (8 pieces,
// two rows per 256 bytes of banks) by (row >> 1) & 7.
template <bool F8>
__device__ __forceinline__ int idx_swz(int row, int piece) {
    return F8 ? piece ^ ((row >> 1) & 7) : piece ^ (row & 15);
}

template <bool V>
struct BoolTag {
    static constexpr bool value = V;
};

// Running top-KC of one row in registers, for blocks offered in ascending id
// order: ts/tb are sorted by score, descending; a new block goes after every
// kept block of equal score (a lower id ranks first). Branch-free: slot i
// keeps its entry, takes the new one, or takes slot i-1's old entry.
template <int KC>
__device__ __forceinline__ void topk_insert(float (&ts)[KC], int (&tb)[KC], float xs, int xb) {
#pragma unroll
    for (int i = KC - 1; i >= 0; --i) {
        const bool keep = ts[i] >= xs;
        const bool prev_ge = i == 0 || ts[i > 0 ? i - 1 : 0] >= xs;
        const float ps = i > 0 ? ts[i - 1] : xs;
        const int pb = i > 0 ? tb[i - 1] : xb;
        ts[i] = keep ? ts[i] : (prev_ge ? xs : ps);
        tb[i] = keep ? tb[i] : (prev_ge ? xb : pb);
    }
}

// KC = 0: pooled block scores are written out. KC = 16 or 32: every lane owns
// one row, keeps its top-KC blocks in registers while the blocks stream by,
// and writes sel / sel_scores (first K) at the end; no pooled scores.
// QB (query-block-shared selection, KC > 0): the workgroup holds one query
// block (the rows of the call at positions qblk*S .. qblk*S+S-1) for two groups,
// waves 2h and 2h+1 the block's first and second 64 rows of group 2*gp + h.
// A key block's score is the largest block max over those rows: a wave
// reduction, then the two waves' values meet in LDS at the next block's
// barrier, where the even wave (every lane alike) offers the block to its
// running top-KC; sel is [B, nslots, G, K] with slot = qblk - floor(q_start/S).
template <bool F8, int KC, bool QB = false>
__global__ __launch_bounds__(256, 2) void idx_prefill_kernel(
    const unsigned char *__restrict__ q_idx, const unsigned char *__restrict__ k_idx,
    const int32_t *__restrict__ kv_lens, const int32_t *__restrict__ q_start,
    float *__restrict__ pooled, int T, int G, int Nmax, int64_t nb_max, int K,
    int32_t *__restrict__ sel, float *__restrict__ sel_scores, int nslots = 0,
    int blk_split = 0) {
    constexpr int kRowBytes = DI * (F8 ? 1 : 2);
    constexpr int kRowPieces = kRowBytes / 16;
    constexpr int kRuns = S * kRowBytes / 1024 / 4;  // 1 KiB staging loads per wave per block
    constexpr int kKs = F8 ? 2 : 8;                  // MFMA K steps over the index dim
    __shared__ __attribute__((aligned(1024))) unsigned char lds_buf[2][S * kRowBytes];
    const int b = blockIdx.y;
    const int rows = T * G;
    const int xr = gridDim.x - 1 - blockIdx.x;  // longest rows first
    const int r0 = xr * kPfRows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    // QB: query block qblk (slot xr / npairs), groups 2*gp and 2*gp + 1.
    const int npairs = (G + 1) / 2;
    const int qblk = QB ? floor_div(qs, S) + xr / npairs : 0;
    const int gp = QB ? xr % npairs : 0;
    int p_lo, p_hi;
    if constexpr (QB) {
        p_lo = max(max(qblk * S, qs), 0);
        p_hi = min(min(qblk * S + S - 1, qs + T - 1), kv - 1);
    } else {
        const int r_last = min(r0 + kPfRows, rows) - 1;
        p_hi = min(qs + r_last / G, kv - 1);
        p_lo = qs + r0 / G;
    }
    if (KC == 0 && p_hi < 0) return;
    const int nblk = (p_hi >= 0 && p_hi >= p_lo) ? p_hi / S + 1 : 0;
    // Pooled scores only: workgroup z of a row tile takes key blocks
    // [z * blk_split, (z + 1) * blk_split) (every block has one writer).
    const int blo = KC == 0 && blk_split > 0 ? (int)blockIdx.z * blk_split : 0;
    const int bhi = KC == 0 && blk_split > 0 ? min(nblk, blo + blk_split) : nblk;
    if (KC == 0 && blo >= bhi) return;

    const int j = lane & 31, half = lane >> 5;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    // B operand: query row (r0 + 64*wave + 32*ct + j); K step ks covers key
    // bytes [ks*kKb, ks*kKb + kKb) of which this lane holds half `half`.
    constexpr int kKb = F8 ? 64 : 32;
    u32x4 qb[2][kKs][F8 ? 2 : 1];
    int pcol[2];
    const int my_g = QB ? 2 * gp + (wave >> 1) : 0;  // QB: this wave's group
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        int r, p;
        bool ok;
        if constexpr (QB) {
            p = qblk * S + 64 * (wave & 1) + 32 * ct + j;
            const int t = p - qs;
            r = t * G + my_g;
            ok = my_g < G && t >= 0 && t < T && p >= 0 && p < kv;
        } else {
            r = r0 + 64 * wave + 32 * ct + j;
            p = qs + r / G;
            ok = r < rows && p >= 0 && p < kv;
        }
        pcol[ct] = ok ? p : -1;
        const unsigned char *qp = q_idx + ((size_t)b * rows + (ok ? r : 0)) * kRowBytes;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
            for (int h = 0; h < (F8 ? 2 : 1); ++h)
                qb[ct][ks][h] = ok ? ld16(qp + ks * kKb + half * (kKb / 2) + 16 * h) : zero4;
    }
    constexpr int KCS = KC > 0 ? KC : 1;
    float ts[KCS];
    int tb[KCS];
#pragma unroll
    for (int i = 0; i < KCS; ++i) {
        ts[i] = -INFINITY;
        tb[i] = -1;
    }
    const unsigned char *kseq = k_idx + (size_t)b * Nmax * kRowBytes;
    // Stage block blk into buffer `buf`: wave w loads 1 KiB runs w, w + 4, ...
    // of the tile; lane l fills physical slot l % kRowPieces of row
    // run * (1024 / kRowBytes) + l / kRowPieces. Loads are clamped to the last
    // key (kv >= 1 whenever a block exists); keys past kv lie past every row's
    // position and are masked.
    auto stage = [&](int blk, unsigned char *buf) {
#pragma unroll
        for (int i = 0; i < kRuns; ++i) {
            const int run = wave + 4 * i;
            const int row = run * (1024 / kRowBytes) + lane / kRowPieces;
            const int piece = idx_swz<F8>(row, lane % kRowPieces);
            const int tok = min(blk * S + row, kv - 1);
            __builtin_amdgcn_global_load_lds(
                (const void *)(kseq + (size_t)tok * kRowBytes + piece * 16),
                (__attribute__((address_space(3))) void *)(buf + run * 1024), 16, 0, 0);
        }
    };
    // QB: the wave's value for the last block, and the two waves' values of
    // the previous two blocks (one LDS pair per block parity).
    __shared__ float s_qb[2][4];
    float qb_own = -INFINITY;
    auto qb_offer = [&](int blk_prev) {  // after a barrier: block blk_prev's score
        if (wave & 1) return;
        const float sc = fmaxf(qb_own, s_qb[blk_prev & 1][wave + 1]) + 0.0f;
        if (sc > ts[KCS - 1]) topk_insert<KCS>(ts, tb, sc, blk_prev);
    };
    // One block: stage it in LDS, prefetch the next, score it, then block max
    // and top-K insertion. MASK: the block reaches past the first row's
    // position, so keys past each row's position are masked; the blocks
    // before that take a plain max (two separate loops, so each is compiled
    // without the other's epilogue).
    auto do_block = [&](auto mask_tag, int blk) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int tok0 = blk * S;
        // This wave's staging loads of block blk have landed (vmcnt(0)) and its
        // LDS reads of block blk - 1 are done (lgkmcnt(0)); after the barrier
        // every wave's have, so blk is complete in its buffer and the other
        // buffer is free for blk + 1.
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if constexpr (QB)
            if (blk > 0) qb_offer(blk - 1);
        if (blk + 1 < bhi) stage(blk + 1, lds_buf[(blk + 1) & 1]);
        const unsigned char *lds = lds_buf[blk & 1];
        float cm0 = -INFINITY, cm1 = -INFINITY;
        // Two row tiles at a time: four independent accumulator chains.
#pragma unroll
        for (int rp = 0; rp < 2; ++rp) {
            f32x16 acc[2][2] = {};
            if constexpr (!F8) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int rt = 2 * rp + h2;
                    // Logical bytes ks*kKb + half*kKb/2 of row rt*32 + j.
                    const int row = rt * 32 + j;
                    const int p0 = (ks * kKb + half * (kKb / 2)) / 16;
                    const unsigned char *ap = lds + row * kRowBytes + idx_swz<F8>(row, p0) * 16;
                    if constexpr (F8) {
                        const unsigned char *ap1 = lds + row * kRowBytes + idx_swz<F8>(row, p0 + 1) * 16;
                        const i32x8 a = cat_i32x8(*reinterpret_cast<const u32x4 *>(ap),
                                                  *reinterpret_cast<const u32x4 *>(ap1));
                        acc[h2][0] = mfma32_f8(a, cat_i32x8(qb[0][ks][0], qb[0][ks][F8 ? 1 : 0]), acc[h2][0]);
                        acc[h2][1] = mfma32_f8(a, cat_i32x8(qb[1][ks][0], qb[1][ks][F8 ? 1 : 0]), acc[h2][1]);
                    } else {
                        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(ap));
                        acc[h2][0] = mfma32(a, as_bf16x8(qb[0][ks][0]), acc[h2][0]);
                        acc[h2][1] = mfma32(a, as_bf16x8(qb[1][ks][0]), acc[h2][1]);
                    }
                }
            }
            // bf16: the row tiles' operand reads run ahead of the MFMAs, two
            // products per read after the first four reads.
            if constexpr (!F8) {
#pragma unroll
                for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                for (int i = 0; i < 2 * kKs - 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int rt = 2 * rp + h2;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float s0 = acc[h2][0][i], s1 = acc[h2][1][i];
                    if constexpr (MASK) {
                        const int tok = tok0 + rt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                        if (tok > pcol[0]) s0 = -INFINITY;
                        if (tok > pcol[1]) s1 = -INFINITY;
                    }
                    cm0 = fmaxf(cm0, s0);
                    cm1 = fmaxf(cm1, s1);
                }
            }
        }
        cm0 = fmaxf(cm0, __shfl_xor(cm0, 32));
        cm1 = fmaxf(cm1, __shfl_xor(cm1, 32));
        const float v = (half ? cm1 : cm0) + 0.0f;
        const int pc = half ? pcol[1] : pcol[0];
        if constexpr (KC == 0) {
            const int r = r0 + 64 * wave + 32 * half + j;
            if (pc >= tok0) pooled[((size_t)b * rows + r) * nb_max + blk] = v;
        } else if constexpr (QB) {
            // The wave's largest block max over its rows that reach the block;
            // the partner wave's value is read after the next barrier.
            float wv = pc >= tok0 ? v : -INFINITY;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) wv = fmaxf(wv, __shfl_xor(wv, off));
            qb_own = wv;
            if (lane == 0) s_qb[blk & 1][wave] = wv;
        } else {
            const bool offer = pc >= tok0 && v > ts[KC - 1];
            if (__ballot(offer)) {
                if (offer) topk_insert<KC>(ts, tb, v, blk);
            }
        }
    };
    // Blocks [0, n_plain) end at or before the first row's position.
    const int n_plain = p_lo >= 0 ? min((p_lo + 1) / S, nblk) : 0;
    if (bhi > blo) stage(blo, lds_buf[blo & 1]);
    for (int blk = blo; blk < min(n_plain, bhi); ++blk) do_block(BoolTag<false>{}, blk);
    for (int blk = max(n_plain, blo); blk < bhi; ++blk) do_block(BoolTag<true>{}, blk);
    if constexpr (QB) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        if (nblk > 0) qb_offer(nblk - 1);
        const int slot = qblk - floor_div(qs, S);
        if ((wave & 1) == 0 && my_g < G && lane == 0 && slot >= 0 && slot < nslots) {
            const size_t o = (((size_t)b * nslots + slot) * G + my_g) * K;
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                if (i < K) {
                    sel[o + i] = tb[i];
                    if (sel_scores) sel_scores[o + i] = ts[i];
                }
            }
        }
    } else if constexpr (KC > 0) {
        const int r = r0 + 64 * wave + 32 * half + j;
        if (r < rows) {
            const size_t o = ((size_t)b * rows + r) * K;
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                if (i < K) {
                    sel[o + i] = tb[i];
                    if (sel_scores) sel_scores[o + i] = ts[i];
                }
            }
        }
    }
}

// Prefill: one 4-wave workgroup per (row, group); wave w takes chunk w of
// every kept block, so a block is read once per workgroup.
struct PrefillLds {
    unsigned char vrows[4 * kVWave];  // V chunks; then the [4][16][128] fp32 wave outputs
    int sel[KMAX];
    int blocks[KMAX];
    int nblk;
    float m[4 * 16], l[4 * 16];
};

__global__ __launch_bounds__(256) void sparse_attn_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache,
    const bf16_t *__restrict__ v_cache, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const int32_t *__restrict__ sel, int T, int G, int R,
    int Nmax, int K, float scale_log2, bf16_t *__restrict__ out, float *__restrict__ lse) {
    __shared__ PrefillLds L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t unit = blockIdx.x;  // (row, group)
    const int g = (int)(unit % G);
    const int64_t bt = unit / G;
    const int b = (int)(bt / T), t = (int)(bt % T);
    const int H = G * R;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int p = qs + t;
    const bool row_ok = p >= 0 && p < kv;
    if (tid < K) L.sel[tid] = row_ok ? sel[unit * K + tid] : -1;
    __syncthreads();
    if (wave == 0) {
        const int n = build_block_list(L.sel, K, row_ok ? p : -1, L.blocks, lane);
        if (lane == 0) L.nblk = n;
    }
    __syncthreads();
    const int nblk = L.nblk;
    bf16x8 qf[4];
    load_query(qf, q + (bt * H + (int64_t)g * R) * D, R, lane);
    const bf16_t *kg_base = k_cache + ((size_t)b * G + g) * Nmax * D;
    const bf16_t *vg_base = v_cache + ((size_t)b * G + g) * Nmax * D;
    WaveAttn st;
    wave_attn_init(st);
    for (int c = 0; c < nblk; ++c)
        attend_chunk(st, qf, kg_base, vg_base, L.blocks[c] * S + wave * 32, p, scale_log2,
                     L.vrows + wave * kVWave, lane);
    merge_and_store<4>(st, R, L.m, L.l, reinterpret_cast<float *>(L.vrows),
                       out + (bt * H + (int64_t)g * R) * D, lse ? lse + bt * H + (int64_t)g * R : nullptr);
}

// ---------------------------------------------------------------------------
// Sparse prefill, KV-major. The dev.to summary of the M3 design (section 二)
// makes the KV tile the outer loop: a tile is read once and serves every query
// that needs it; [T] §六 has all heads of a group share the kept blocks. Here
// a kept block of one group is staged in LDS once per workgroup and every
// (row, head) that kept it attends over it there. Per pass of `rows` query
// rows of every sequence:
//   list build        each kept (row, group, slot) goes into the list of its
//                     (sequence, group, block), in row order (the kernels
//                     below build_pass_lists: a bitmap per list, its prefix
//                     popcounts, offsets and tiles of CH entries, scatter);
//   pf_attn_kernel    one workgroup per tile: K and V of the block in LDS,
//                     then R heads per entry attend over its 128 keys
//                     (16x16x32 MFMA, the chunk step of attend_chunk with
//                     kPfNq query tiles per wave), writing a normalised partial
//                     (O / l in bf16, m and l in fp32) per (row, group, slot);
//   pf_merge_kernel   one workgroup per (row, group): log-sum-exp merge of the
//                     kept slots' partials into out and lse.
// A slot is kept when its block id is a causal block of the row (0 <= id <=
// p/S) and no earlier slot of the row holds the same id. The forward's results
// do not depend on the list order (every partial has its own place); the
// backward's dk and dv sum over the lists, so the order is fixed.
constexpr int kKRow = 272;  // staged K row bytes: 256 + 16 pad
constexpr int kPfWaves = msa::kPfWaves;
constexpr int kPfNq = msa::kPfNq;
// Most entries of one tile (R = 1): entries_per_tile * R is the same for all R.
constexpr int kPfTileEntriesMax = msa::kPfRounds * msa::kPfWaves * msa::kPfNq * 16;


// One wavefront per new (sequence, row): the row's G K rows and G V rows
// (256 B each) and its index key (kib bytes) are copied 16 B per lane.
__global__ __launch_bounds__(256) void cache_append_kernel(
    const u32x4 *__restrict__ k_new, const u32x4 *__restrict__ v_new,
    const unsigned char *__restrict__ ki_new, const int32_t *__restrict__ pos0, int B, int T,
    int G, int Nmax, int kib, u32x4 *__restrict__ k_cache, u32x4 *__restrict__ v_cache,
    unsigned char *__restrict__ k_idx) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * T + t
    if (row >= (int64_t)B * T) return;
    const int b = (int)(row / T), t = (int)(row % T);
    const int64_t pos = (int64_t)pos0[b] + t;
    if (pos < 0 || pos >= Nmax) return;
    constexpr int kPieces = D * 2 / 16;  // 16-byte pieces per K or V row
    for (int i = lane; i < G * kPieces; i += 64) {
        const int g = i / kPieces, c = i % kPieces;
        const int64_t dst = (((int64_t)b * G + g) * Nmax + pos) * kPieces + c;
        k_cache[dst] = k_new[row * G * kPieces + i];
        v_cache[dst] = v_new[row * G * kPieces + i];
    }
    const int ki_pieces = kib / 16;
    if (lane < ki_pieces)
        reinterpret_cast<u32x4 *>(k_idx + ((int64_t)b * Nmax + pos) * kib)[lane] =
            reinterpret_cast<const u32x4 *>(ki_new + row * kib)[lane];
}


// List build of a pass: a counting sort of the kept (row, group, slot)
// entries by block that keeps row order inside every list, so lists and tiles
// come out the same on every run (the backward sums over them):
//   pf_clear_kernel    zeroes the row bitmaps of the lists that can hold
//                      entries (not launched for caches of at most
//                      kPfMarkAllBlocks blocks, whose marking stores every
//                      word);
//   pf_mark_lds_kernel (caches of up to kPfMarkLdsBlocks blocks) or
//   pf_mark_kernel     sets bit tl of the kept block's row bitmap (an OR in
//                      LDS per 32 rows, then a plain store per nonzero word;
//                      or a global atomic OR; either result is order-free);
//   pf_rank_kernel     per list: exclusive prefix popcounts of its bitmap
//                      words and its entry count;
//   pf_scan_small_kernel (up to kScanSmall lists) or
//   pf_scan_kernel     list offsets and tiles;
//   pf_scatter_lds_kernel (with pf_mark_lds_kernel) or
//   pf_scatter_kernel  an entry's rank is its word's prefix plus the popcount
//                      of the lower bits of its word (rebuilt in LDS, or read).
// Thread per (sequence, row of the pass, group, slot).
__global__ __launch_bounds__(256) void pf_mark_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, int B, int T, int G, int Nmax, int K, int t0, int rows,
    int g0, int ng, int64_t nb_max, int W, uint32_t *__restrict__ bits) {
    const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (slot >= (int64_t)B * rows * ng * K) return;
    const int k = (int)(slot % K);
    const int64_t unit = slot / K;  // (b, tl, gl), group g0 + gl
    const int gl = (int)(unit % ng);
    const int64_t btl = unit / ng;
    const int b = (int)(btl / rows), tl = (int)(btl % rows);
    const int t = t0 + tl;
    const int p = pf_row_pos(kv_lens, q_start, b, t, T, Nmax);
    if (p < 0) return;
    const int32_t *sr = sel + (((int64_t)b * T + t) * G + g0 + gl) * K;
    if (!slot_kept(sr, k, p / S + 1)) return;
    const int64_t li = ((int64_t)b * ng + gl) * nb_max + sr[k];
    atomicOr(&bits[li * W + (tl >> 5)], 1u << (tl & 31));
}

// Key blocks of sequence b that exist (any row's kept blocks lie below):
// lists (b, group, block) at or past it stay empty, so the list build
// neither clears nor ranks their bitmaps (a chunk early in a long cache has
// most of its lists past the keys written so far).
__device__ __forceinline__ int pf_key_blocks(const int32_t *kv_lens, int b, int Nmax) {
    const int kv = clamp_kv(kv_lens[b], Nmax);
    return kv > 0 ? (kv - 1) / S + 1 : 0;
}

// Marking without global atomics, for caches of at most kPfMarkLdsBlocks key
// blocks: workgroup per (sequence, 32 rows of the pass = one bitmap word,
// group). Its rows' kept blocks set their bits in an LDS word per key block
// (LDS OR), then every nonzero word goes to bits[list][word] with a plain
// store: that word of every list belongs to this workgroup alone, and
// pf_clear_kernel has zeroed the rest. With write_all (caches of at most
// kPfMarkAllBlocks blocks, where the scattered zero stores are few) every
// word below the key blocks is stored and no clear runs.
constexpr int kPfMarkLdsBlocks = 16384;
constexpr int kPfMarkAllBlocks = 64;
__global__ __launch_bounds__(256) void pf_mark_lds_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, int T, int G, int Nmax, int K, int t0, int rows,
    int g0, int ng, int64_t nb_max, int W, int write_all, uint32_t *__restrict__ bits) {
    // Dynamic LDS: nb_max words, then the 32 rows' selections (32 * K).
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];
    uint32_t *s_word = s_dyn;
    int32_t *s_sel = reinterpret_cast<int32_t *>(s_dyn + nb_max);
    const int tid = threadIdx.x;
    const int gl = (int)(blockIdx.x % (unsigned)ng);
    const int bc = (int)(blockIdx.x / (unsigned)ng);  // (b, word c)
    const int b = bc / W, c = bc % W;
    const int nb = pf_key_blocks(kv_lens, b, Nmax);
    const int r0 = 32 * c, nr = min(32, rows - r0);
    for (int i = tid; i < nb; i += 256) s_word[i] = 0u;
    for (int i = tid; i < nr * K; i += 256) {
        const int t = t0 + r0 + i / K;  // a last pass may reach past the call's rows
        s_sel[i] = t < T ? sel[(((int64_t)b * T + t) * G + g0 + gl) * K + i % K] : -1;
    }
    __syncthreads();
    for (int i = tid; i < nr * K; i += 256) {
        const int rl = i / K, k = i % K;
        const int p = pf_row_pos(kv_lens, q_start, b, t0 + r0 + rl, T, Nmax);
        if (p < 0 || !slot_kept(s_sel + rl * K, k, p / S + 1)) continue;
        atomicOr(&s_word[s_sel[i]], 1u << rl);  // kept ids lie below p / S + 1 <= nb
    }
    __syncthreads();
    uint32_t *col = bits + ((int64_t)b * ng + gl) * nb_max * W + c;
    for (int i = tid; i < nb; i += 256) {
        const uint32_t v = s_word[i];
        if (v || write_all) col[(int64_t)i * W] = v;
    }
}

// Workgroup per (list, 1024 words of its bitmap): zero the words of the
// lists that can hold entries (the list's coordinates are workgroup-uniform).
__global__ __launch_bounds__(256) void pf_clear_kernel(uint32_t *__restrict__ bits,
                                                       const int32_t *__restrict__ kv_lens,
                                                       int W, int wchunks, int ng,
                                                       int64_t nb_max, int Nmax) {
    const int64_t li = blockIdx.x / (unsigned)wchunks;
    const int w0 = (int)(blockIdx.x % (unsigned)wchunks) * 1024;
    const int b = (int)(li / ((int64_t)ng * nb_max));
    if (li % nb_max >= pf_key_blocks(kv_lens, b, Nmax)) return;
    uint32_t *row = bits + li * W;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int w = w0 + u * 256 + (int)threadIdx.x;
        if (w < W) row[w] = 0u;
    }
}

// Wave per list.
__global__ __launch_bounds__(256) void pf_rank_kernel(const uint32_t *__restrict__ bits,
                                                      int64_t nlists, int W,
                                                      const int32_t *__restrict__ kv_lens,
                                                      int ng, int64_t nb_max, int Nmax,
                                                      int32_t *__restrict__ wpre,
                                                      int32_t *__restrict__ counts) {
    const int64_t li = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (li >= nlists) return;
    const int b = (int)(li / ((int64_t)ng * nb_max));
    if (li % nb_max >= pf_key_blocks(kv_lens, b, Nmax)) {  // no entries; words never read
        if (lane == 0) counts[li] = 0;
        return;
    }
    const uint32_t *bw = bits + li * W;
    int32_t *pw = wpre + li * W;
    int run = 0;
    for (int w0 = 0; w0 < W; w0 += 64) {
        const int i = w0 + lane;
        const int c = i < W ? __popc(bw[i]) : 0;
        int x = c;  // inclusive scan over the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (i < W) pw[i] = run + x - c;
        run += __shfl(x, 63);
    }
    if (lane == 0) counts[li] = run;
}

// One workgroup of 1024 threads: exclusive scans of the list sizes and of
// their tile counts, and the tile -> list map. The lists go by in segments
// of 8192: the segment's sizes are read coalesced into LDS, every thread
// takes eight consecutive ones, a workgroup scan places them after the
// previous segments, and the offsets and tile starts are written back
// coalesced from LDS (the tile map directly).
constexpr int kScanSeg = 8;  // lists per thread per segment
__global__ __launch_bounds__(1024) void pf_scan_kernel(const int32_t *__restrict__ counts,
                                                       int64_t n, int ch,
                                                       int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ tile_first,
                                                       int32_t *__restrict__ tile_map) {
    constexpr int kSeg = 1024 * kScanSeg;
    __shared__ int32_t s_c[kSeg], s_f[kSeg];
    __shared__ int32_t s_e[1024], s_t[1024];
    const int tid = threadIdx.x;
    int32_t base_e = 0, base_t = 0;  // totals of the previous segments
    for (int64_t s0 = 0; s0 < n; s0 += kSeg) {
        const int m = (int)min((int64_t)kSeg, n - s0);
#pragma unroll
        for (int v = 0; v < kScanSeg; ++v) {
            const int i = v * 1024 + tid;
            s_c[i] = i < m ? counts[s0 + i] : 0;
        }
        __syncthreads();
        int32_t c[kScanSeg], nt[kScanSeg], se = 0, st = 0;
#pragma unroll
        for (int u = 0; u < kScanSeg; ++u) {
            c[u] = s_c[tid * kScanSeg + u];
            nt[u] = (c[u] + ch - 1) / ch;
            se += c[u];
            st += nt[u];
        }
        s_e[tid] = se;
        s_t[tid] = st;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t ve = tid >= off ? s_e[tid - off] : 0;
            const int32_t vt = tid >= off ? s_t[tid - off] : 0;
            __syncthreads();
            s_e[tid] += ve;
            s_t[tid] += vt;
            __syncthreads();
        }
        int32_t oe = base_e + s_e[tid] - se, ot = base_t + s_t[tid] - st;
#pragma unroll
        for (int u = 0; u < kScanSeg; ++u) {
            const int i = tid * kScanSeg + u;
            s_c[i] = oe;  // this thread's own entries: no other thread reads them now
            s_f[i] = ot;
            if (i < m)
                for (int32_t j = 0; j < nt[u]; ++j) tile_map[ot + j] = (int32_t)(s0 + i);
            oe += c[u];
            ot += nt[u];
        }
        base_e += s_e[1023];
        base_t += s_t[1023];
        __syncthreads();
#pragma unroll
        for (int v = 0; v < kScanSeg; ++v) {
            const int i = v * 1024 + tid;
            if (i < m) {
                offsets[s0 + i] = s_c[i];
                tile_first[s0 + i] = s_f[i];
            }
        }
        __syncthreads();  // s_c, s_e and s_t are refilled by the next segment
    }
    if (tid == 0) {
        offsets[n] = base_e;
        tile_first[n] = base_t;
    }
}

// The same scan for at most kScanSmall lists: every thread walks a run of
// consecutive lists (for a few dozen lists, as in short prefills, this is
// several times faster than the segmented form). The runs' sums are scanned
// within each wave by lane shuffles, then the sixteen wave totals by wave 0:
// two barriers.
constexpr int64_t kScanSmall = 8192;
__global__ __launch_bounds__(1024) void pf_scan_small_kernel(const int32_t *__restrict__ counts,
                                                       int64_t n, int ch,
                                                       int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ tile_first,
                                                       int32_t *__restrict__ tile_map) {
    __shared__ int32_t s_we[16], s_wt[16], s_tot[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t per = (n + 1023) / 1024;
    const int64_t a = min(n, (int64_t)tid * per), e = min(n, a + per);
    // A thread's list sizes are read kBatch at a time, in both walks.
    constexpr int kBatch = 16;
    int32_t se = 0, st = 0;
    for (int64_t i0 = a; i0 < e; i0 += kBatch) {
        int32_t c[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) c[u] = i0 + u < e ? counts[i0 + u] : 0;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            se += c[u];
            st += (c[u] + ch - 1) / ch;
        }
    }
    int32_t xe = se, xt = st;  // inclusive scans over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t ye = __shfl_up(xe, off), yt = __shfl_up(xt, off);
        if (lane >= off) {
            xe += ye;
            xt += yt;
        }
    }
    if (lane == 63) {
        s_we[wave] = xe;
        s_wt[wave] = xt;
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefixes of the wave totals, and the totals
        const int32_t we = lane < 16 ? s_we[lane] : 0, wt = lane < 16 ? s_wt[lane] : 0;
        int32_t ve = we, vt = wt;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int32_t ye = __shfl_up(ve, off), yt = __shfl_up(vt, off);
            if (lane >= off) {
                ve += ye;
                vt += yt;
            }
        }
        if (lane < 16) {
            s_we[lane] = ve - we;
            s_wt[lane] = vt - wt;
        }
        if (lane == 15) {
            s_tot[0] = ve;
            s_tot[1] = vt;
        }
    }
    __syncthreads();
    int32_t oe = s_we[wave] + xe - se, ot = s_wt[wave] + xt - st;
    for (int64_t i0 = a; i0 < e; i0 += kBatch) {
        int32_t c[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) c[u] = i0 + u < e ? counts[i0 + u] : 0;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t i = i0 + u;
            if (i < e) {
                const int32_t nt = (c[u] + ch - 1) / ch;
                offsets[i] = oe;
                tile_first[i] = ot;
                for (int32_t j = 0; j < nt; ++j) tile_map[ot + j] = (int32_t)i;
                oe += c[u];
                ot += nt;
            }
        }
    }
    if (tid == 0) {
        offsets[n] = s_tot[0];
        tile_first[n] = s_tot[1];
    }
}

// The scatter for caches of up to kPfMarkLdsBlocks key blocks, on the grid
// of pf_mark_lds_kernel: the workgroup rebuilds its bitmap word of every list
// in LDS (the same OR), so an entry's rank needs only its word's prefix.
__global__ __launch_bounds__(256) void pf_scatter_lds_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const int32_t *__restrict__ wpre,
    const int32_t *__restrict__ offsets, int T, int G, int Nmax, int K, int t0, int rows,
    int g0, int ng, int64_t nb_max, int W, int32_t *__restrict__ list) {
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];
    uint32_t *s_word = s_dyn;
    int32_t *s_sel = reinterpret_cast<int32_t *>(s_dyn + nb_max);
    const int tid = threadIdx.x;
    const int gl = (int)(blockIdx.x % (unsigned)ng);
    const int bc = (int)(blockIdx.x / (unsigned)ng);  // (b, word c)
    const int b = bc / W, c = bc % W;
    const int nb = pf_key_blocks(kv_lens, b, Nmax);
    const int r0 = 32 * c, nr = min(32, rows - r0);
    for (int i = tid; i < nb; i += 256) s_word[i] = 0u;
    for (int i = tid; i < nr * K; i += 256) {
        const int t = t0 + r0 + i / K;
        s_sel[i] = t < T ? sel[(((int64_t)b * T + t) * G + g0 + gl) * K + i % K] : -1;
    }
    __syncthreads();
    // Kept entries: this thread's, as a bit mask over its (at most eight) indices.
    uint32_t mine = 0u;
    for (int i = tid, n = 0; i < nr * K; i += 256, ++n) {
        const int rl = i / K, k = i % K;
        const int p = pf_row_pos(kv_lens, q_start, b, t0 + r0 + rl, T, Nmax);
        if (p < 0 || !slot_kept(s_sel + rl * K, k, p / S + 1)) continue;
        mine |= 1u << n;
        atomicOr(&s_word[s_sel[i]], 1u << rl);
    }
    __syncthreads();
    const int64_t l0 = ((int64_t)b * ng + gl) * nb_max;
    for (int i = tid, n = 0; i < nr * K; i += 256, ++n) {
        if (!((mine >> n) & 1u)) continue;
        const int rl = i / K, k = i % K;
        const int blk = s_sel[i];
        const int64_t li = l0 + blk;
        const int r = wpre[li * W + c] + __popc(s_word[blk] & ((1u << rl) - 1u));
        list[offsets[li] + r] = ((r0 + rl) << kEntShift) | k;
    }
}

__global__ __launch_bounds__(256) void pf_scatter_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const uint32_t *__restrict__ bits,
    const int32_t *__restrict__ wpre, const int32_t *__restrict__ offsets, int B, int T, int G,
    int Nmax, int K, int t0, int rows, int g0, int ng, int64_t nb_max, int W,
    int32_t *__restrict__ list) {
    const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (slot >= (int64_t)B * rows * ng * K) return;
    const int k = (int)(slot % K);
    const int64_t unit = slot / K;
    const int gl = (int)(unit % ng);
    const int64_t btl = unit / ng;
    const int b = (int)(btl / rows), tl = (int)(btl % rows);
    const int t = t0 + tl;
    const int p = pf_row_pos(kv_lens, q_start, b, t, T, Nmax);
    if (p < 0) return;
    const int32_t *sr = sel + (((int64_t)b * T + t) * G + g0 + gl) * K;
    if (!slot_kept(sr, k, p / S + 1)) return;
    const int64_t li = ((int64_t)b * ng + gl) * nb_max + sr[k];
    const int64_t wi = li * W + (tl >> 5);
    const int r = wpre[wi] + __popc(bits[wi] & ((1u << (tl & 31)) - 1u));
    list[offsets[li] + r] = (tl << kEntShift) | k;
}

__global__ __launch_bounds__(256, 2) void pf_attn_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache,
    const bf16_t *__restrict__ v_cache, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ tile_first, const int32_t *__restrict__ tile_map,
    const int32_t *__restrict__ list, int64_t nlists, int T, int G, int R, int Nmax, int K,
    int t0, int rows, int g0, int ng, int64_t nb_max, int ch, float scale_log2,
    bf16_t *__restrict__ part_o, float2 *__restrict__ part_ml, unsigned char *__restrict__ trash) {
    __shared__ __attribute__((aligned(16))) unsigned char k_lds[S * kKRow];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[S * kVRow];
    __shared__ int s_ent[kPfTileEntriesMax];  // the tile's list entries
    const int w = blockIdx.x;
    if (w >= tile_first[nlists]) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kg = lane >> 4;
    const int li = tile_map[w];
    const int beg = offsets[li] + (w - tile_first[li]) * ch;
    const int nent = min(beg + ch, offsets[li + 1]) - beg;
    if (nent <= 0) return;
    const int64_t bgl = li / nb_max;  // (sequence, group of the pass)
    const int blk = (int)(li % nb_max);
    const int b = (int)(bgl / ng), gl = (int)(bgl % ng), g = g0 + gl;
    const int64_t bg = (int64_t)b * G + g;
    const int H = G * R;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    // Stage the block: 128 K rows and 128 V rows of 256 bytes, zero past kv.
    {
        const bf16_t *kb = k_cache + (bg * Nmax + (int64_t)blk * S) * D;
        const bf16_t *vb = v_cache + (bg * Nmax + (int64_t)blk * S) * D;
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        u32x4 kr[8], vr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int piece = tid + 256 * i, tk = piece >> 4, c = piece & 15;
            const bool in = blk * S + tk < kv;
            kr[i] = in ? ld16(kb + (size_t)tk * D + c * 8) : z4;
            vr[i] = in ? ld16(vb + (size_t)tk * D + c * 8) : z4;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int piece = tid + 256 * i, tk = piece >> 4, c = piece & 15;
            *reinterpret_cast<u32x4 *>(k_lds + tk * kKRow + c * 16) = kr[i];
            *reinterpret_cast<u32x4 *>(v_lds + tk * kVRow + c * 16) = vr[i];
        }
        for (int i = tid; i < nent; i += 256) s_ent[i] = list[beg + i];
    }
    __syncthreads();
    const int et = 16 / R;  // entries per 16-column query tile
    const int tok_base = blk * S;
    // Column `col` of query tile nq in a round: entry e0 + nq*et + col/R, head
    // col%R. Two register sets alternate between rounds: right after a round's
    // score MFMAs its set is reloaded with the queries of the round after
    // next, so those loads have about a round and a half to land. The entries
    // come from LDS and a column past the tile's entries loads the last
    // entry's queries (its results are never stored; columns do not mix), so
    // the query loads are unconditional and never wait for the list.
    auto load_round = [&](int e0, int (&ent)[kPfNq], int (&pcol)[kPfNq],
                          bf16x8 (&qf)[kPfNq][4]) {
#pragma unroll
        for (int nq = 0; nq < kPfNq; ++nq) {
            const int e = e0 + nq * et + col / R;
            const bool ok = col < et * R && e < nent;
            const int raw = s_ent[min(e, nent - 1)];
            ent[nq] = ok ? raw : -1;
            const int tl = raw >> kEntShift;
            pcol[nq] = ok ? qs + t0 + tl : -1;
            const bf16_t *qp =
                q + (((int64_t)b * T + t0 + tl) * H + (int64_t)g * R + col % R) * D + kg * 8;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) qf[nq][kc] = ld_bf16x8(qp + kc * 32);
        }
    };
    const int round_step = kPfWaves * kPfNq * et;
    auto do_round = [&](int e0, int (&ent)[kPfNq], int (&pcol)[kPfNq], bf16x8 (&qf)[kPfNq][4]) {
        // S^T for the whole block: key tile kt (16 keys) x 16 query columns;
        // lane holds column `col`, keys kt*16 + 4*kg + r.
        f32x4 sacc[kPfNq][8];
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            // Keeps the scheduler from hoisting every key tile's LDS reads at
            // once (that exhausts the registers).
            if (kt % 2 == 0) __builtin_amdgcn_sched_barrier(0);
            u32x4 ka[4];
            const unsigned char *kp = k_lds + (kt * 16 + col) * kKRow + kg * 16;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) ka[kc] = *reinterpret_cast<const u32x4 *>(kp + kc * 64);
#pragma unroll
            for (int nq = 0; nq < kPfNq; ++nq) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) acc = mfma16(as_bf16x8(ka[kc]), qf[nq][kc], acc);
                sacc[nq][kt] = acc;
            }
        }
        // The queries are no longer needed: reload the set for two rounds on.
        int cent[kPfNq], cpcol[kPfNq];
#pragma unroll
        for (int nq = 0; nq < kPfNq; ++nq) {
            cent[nq] = ent[nq];
            cpcol[nq] = pcol[nq];
        }
        // Unconditional (a step past the tile loads valid rows), so the wait
        // for a round's queries counts the same loads and stores on every
        // path and need not wait for this round's stores.
        load_round(e0 + 2 * round_step, ent, pcol, qf);
        // Softmax over the block's 128 keys in one pass (the block is whole).
        // Only a block that reaches past some column's position is masked.
        bool diag = false;
#pragma unroll
        for (int nq = 0; nq < kPfNq; ++nq) diag |= cent[nq] >= 0 && cpcol[nq] < tok_base + S - 1;
        diag = __ballot(diag) != 0;
        bf16x8 pa[kPfNq][4];
        float mrow[kPfNq], lrow[kPfNq];
#pragma unroll
        for (int nq = 0; nq < kPfNq; ++nq) {
            // Max of the raw scores (the scale is positive), then
            // p = 2^(s*scale - m) with one fma per score.
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float sv = sacc[nq][kt][r];
                    if (diag && tok_base + kt * 16 + 4 * kg + r > cpcol[nq]) sv = -INFINITY;
                    sacc[nq][kt][r] = sv;
                    mx = fmaxf(mx, sv);
                }
            mx = max_xor16_32(mx, lane);
            const float m2 = mx * scale_log2;
            const float neg_m = mx == -INFINITY ? 0.f : -m2;
            float psum = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float pv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    pv[i] = fast_exp2(fmaf(sacc[nq][2 * c + (i >> 2)][i & 3], scale_log2, neg_m));
                    psum += pv[i];
                }
                const u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                  pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
                pa[nq][c] = as_bf16x8(pk);
            }
            psum = sum_xor16_32(psum, lane);
            mrow[nq] = m2;
            lrow[nq] = psum;
        }
        // O^T = V^T x P^T, 32 keys per MFMA step: the V tile read transposed
        // from LDS (same addressing as attend_chunk) is the A operand and the
        // probabilities the B operand, so lane (col, kg) ends up with
        // O[column col][d = dt*16 + 4*kg + r] - four consecutive d per dt.
        f32x4 o[kPfNq][8];
#pragma unroll
        for (int nq = 0; nq < kPfNq; ++nq)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) o[nq][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < S / 32; ++c) {
            const unsigned char *vlo = v_lds + (c * 32 + 4 * kg + (col >> 2)) * kVRow + (col & 3) * 8;
            const unsigned char *vhi = vlo + 16 * kVRow;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                if (dt % 4 == 0) __builtin_amdgcn_sched_barrier(0);
                const u32x2 lo = lds_read_tr16(vlo + dt * 32);
                const u32x2 hi = lds_read_tr16(vhi + dt * 32);
                const u32x4 vbv = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int nq = 0; nq < kPfNq; ++nq) o[nq][dt] = mfma16(as_bf16x8(vbv), pa[nq][c], o[nq][dt]);
            }
        }
        // Partials: m and l of column `col` are in every lane of the column.
        // Lanes kg and kg^1 of a column trade halves (v_permlane16_swap) so
        // that each holds 8 consecutive d-values of two dt steps: lane kg
        // then stores 16 bytes at 64*j + 16*(2*(kg&1) + (kg>>1)) of the
        // head's row, the column's four lanes one 64-byte run per store.
#pragma unroll
        for (int nq = 0; nq < kPfNq; ++nq) {
            const float inv = cent[nq] >= 0 ? 1.f / lrow[nq] : 0.f;
            u32x4 w4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // E: dt = 2j (kept by even kg), O: dt = 2j+1 (kept by odd kg).
                const uint32_t e0 = pack_bf16x2(o[nq][2 * j][0] * inv, o[nq][2 * j][1] * inv);
                const uint32_t e1 = pack_bf16x2(o[nq][2 * j][2] * inv, o[nq][2 * j][3] * inv);
                const uint32_t o0 = pack_bf16x2(o[nq][2 * j + 1][0] * inv, o[nq][2 * j + 1][1] * inv);
                const uint32_t o1 = pack_bf16x2(o[nq][2 * j + 1][2] * inv, o[nq][2 * j + 1][3] * inv);
                const auto r0 = __builtin_amdgcn_permlane16_swap(e0, o0, false, false);
                const auto r1 = __builtin_amdgcn_permlane16_swap(e1, o1, false, false);
                // Even kg: (own E, partner's E); odd kg: (partner's O, own O).
                w4[j] = u32x4{r0[0], r1[0], r0[1], r1[1]};
            }
            // A column without an entry (and the m, l copies of lanes kg > 0)
            // store into the trash area instead of branching around.
            const bool has = cent[nq] >= 0;
            const int64_t slot =
                (((int64_t)b * rows + (cent[nq] >> kEntShift)) * ng + gl) * K +
                (cent[nq] & kEntMask);
            float2 *mlp = has && kg == 0 ? part_ml + slot * R + col % R
                                         : reinterpret_cast<float2 *>(trash + 4096) + col;
            *mlp = make_float2(mrow[nq], lrow[nq]);
            unsigned char *op =
                (has ? reinterpret_cast<unsigned char *>(part_o + (slot * R + col % R) * D)
                     : trash + (col % R) * D * 2) +
                16 * (2 * (kg & 1) + (kg >> 1));
            // Written once, read once by the merge: streaming (nontemporal) stores.
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_nontemporal_store(w4[j], reinterpret_cast<u32x4 *>(op + 64 * j));
        }
    };
    int entA[kPfNq], pcolA[kPfNq], entB[kPfNq], pcolB[kPfNq];
    bf16x8 qA[kPfNq][4], qB[kPfNq][4];
    int e0 = wave * kPfNq * et;
    load_round(e0, entA, pcolA, qA);
    load_round(e0 + round_step, entB, pcolB, qB);
    while (e0 < nent) {
        do_round(e0, entA, pcolA, qA);
        e0 += round_step;
        if (e0 >= nent) break;
        do_round(e0, entB, pcolB, qB);
        e0 += round_step;
    }
}

// Sparse prefill with query-block-shared selections (the mlqm.cn article,
// section 核心原理: 128-token blocks, each attending to its 16 most relevant
// blocks). Every row of query block qblk attends over the same kept blocks,
// so a workgroup keeps 16*et rows' queries (et = 16/R rows per 16-column
// tile, two tiles per wave, eight waves) in registers and streams the unit's
// kept blocks through LDS with an online softmax across blocks: no partials,
// each K/V block staged once per workgroup and used by every column.
//   Staging: direct global->LDS 16-byte loads (lane l of a load fills bytes
// 16l..16l+15 of a 1 KiB run, four 256-byte rows), double-buffered, so block
// i+1 streams in while block i is computed. Rows are unpadded and their
// sixteen 16-byte pieces are XOR-swizzled by the row's low four bits
// (qb_swz), which keeps the K reads (16 rows, same logical piece) on distinct
// banks. Rows past the cache
// are loaded from its last row (finite values that the mask and P = 0 drop).
//   Units are (sequence, slot, group); ncw workgroups split a unit's rows.
// Workgroup ids id, id + 8, ... land on one XCD, so the ncw workgroups of a
// unit (ids 8*(ncw*u') + x + 8*c) share that XCD's L2.
constexpr int kQbWaves = 8;
constexpr float kQbSlack = 8.f;  // log2 units a column's max may exceed its reference
constexpr int kQbBuf = 2 * S * 256;  // K then V of one block, unpadded rows

// Byte offset of logical 16-byte piece `piece` of staged row `row`: the
// piece index is XORed with the row's low four bits, so the 16 rows a K read
// touches (one logical piece) land on 16 different pieces.
__device__ __forceinline__ int qb_swz_key(int row) { return row & 15; }
__device__ __forceinline__ int qb_swz(int row, int piece) {
    return row * 256 + ((piece ^ qb_swz_key(row)) << 4);
}

__global__ __launch_bounds__(512, 1) void qb_attn_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache,
    const bf16_t *__restrict__ v_cache, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const int32_t *__restrict__ sel, int T, int G, int R,
    int Nmax, int K, int nslots, int ncw, int64_t nunits, float scale_log2,
    bf16_t *__restrict__ out, float *__restrict__ lse) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds_kv[2][kQbBuf];
    __shared__ int s_sel[KMAX], s_blocks[KMAX], s_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kg = lane >> 4;
    const int64_t id = blockIdx.x;
    const int64_t unit = (id / 8 / ncw) * 8 + id % 8;
    const int cw = (int)(id / 8 % ncw);
    if (unit >= nunits) return;
    const int g = (int)(unit % G);
    const int64_t bs = unit / G;
    const int slot = (int)(bs % nslots), b = (int)(bs / nslots);
    const int H = G * R;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int qblk = floor_div(qs, S) + slot;
    const int et = 16 / R;
    const int ppw = kQbWaves * kPfNq * et;  // rows (positions) per workgroup
    // Column col of tile nq: position qblk*S + pi, head col % R.
    int trow[kPfNq], pcol[kPfNq];
    bf16x8 qf[kPfNq][4];
#pragma unroll
    for (int nq = 0; nq < kPfNq; ++nq) {
        const int pi = cw * ppw + (wave * kPfNq + nq) * et + col / R;
        const int p = qblk * S + pi;
        const int t = p - qs;
        const bool in_call = col < et * R && pi < S && t >= 0 && t < T;
        const bool valid = in_call && p >= 0 && p < kv;
        trow[nq] = in_call ? t : -1;
        pcol[nq] = valid ? p : -1;
        const bf16_t *qp =
            q + (((int64_t)b * T + (valid ? t : 0)) * H + (int64_t)g * R + col % R) * D + kg * 8;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) qf[nq][kc] = valid ? ld_bf16x8(qp + kc * 32) : zero_bf16x8();
    }
    // The unit's kept blocks: valid ids up to the block of its last row.
    const int p_min = max(max(qblk * S, qs), 0);
    const int p_max = min(min(qblk * S + S - 1, qs + T - 1), kv - 1);
    if (tid < K) s_sel[tid] = sel[(((int64_t)b * nslots + slot) * G + g) * K + tid];
    __syncthreads();
    if (wave == 0) {
        const int n = p_max >= p_min ? build_block_list(s_sel, K, p_max, s_blocks, lane) : 0;
        if (lane == 0) s_n = n;
    }
    __syncthreads();
    const int nblk = s_n;
    const int64_t bg = (int64_t)b * G + g;
    // Wave w stages 1 KiB runs w, w + 8, ... of the 64 KiB (K runs 0..31,
    // V runs 32..63); lane l fills physical piece l & 15 of row 4*run + l/16.
    auto stage = [&](int blk, unsigned char *buf) {
#pragma unroll
        for (int i = 0; i < 2 * S * 256 / 1024 / kQbWaves; ++i) {
            const int run = wave + kQbWaves * i;
            const int kvsel = run >= 32;
            const int row = (run & 31) * 4 + (lane >> 4);
            const int tok = min(blk * S + row, kv - 1);
            const int piece = (lane & 15) ^ qb_swz_key(row);
            const bf16_t *src = (kvsel ? v_cache : k_cache) + (bg * Nmax + tok) * D + piece * 8;
            __builtin_amdgcn_global_load_lds(
                (const void *)src, (__attribute__((address_space(3))) void *)(buf + run * 1024),
                16, 0, 0);
        }
    };
    float m2[kPfNq], lsum[kPfNq];
    f32x4 o[kPfNq][8];
#pragma unroll
    for (int nq = 0; nq < kPfNq; ++nq) {
        m2[nq] = -INFINITY;
        lsum[nq] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[nq][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (nblk > 0) stage(s_blocks[0], lds_kv[0]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's runs (and its queries) landed
    __syncthreads();
    for (int bi = 0; bi < nblk; ++bi) {
        const int blk = s_blocks[bi];
        const int tok_base = blk * S;
        // The next block streams into the other buffer (last read in the
        // previous iteration, before its closing barrier).
        if (bi + 1 < nblk) stage(s_blocks[bi + 1], lds_kv[(bi + 1) & 1]);
        const unsigned char *k_lds = lds_kv[bi & 1];
        const unsigned char *v_lds = k_lds + S * 256;
        // S^T: key tile kt x 16 columns; lane holds column col, keys kt*16 + 4*kg + r.
        f32x4 sacc[kPfNq][8];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            u32x4 ka[4];
            const int row = kt * 16 + col;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                ka[kc] = *reinterpret_cast<const u32x4 *>(k_lds + qb_swz(row, kc * 4 + kg));
#pragma unroll
            for (int nq = 0; nq < kPfNq; ++nq) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) acc = mfma16(as_bf16x8(ka[kc]), qf[nq][kc], acc);
                sacc[nq][kt] = acc;
            }
        }
        // Reads run two key tiles ahead of the products.
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int i = 0; i < 24; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        __builtin_amdgcn_sched_barrier(0);
        // Online softmax across blocks (log2 domain). Only the query block's
        // own key block reaches past a row's position (a uniform branch). The
        // reference m2 moves only when a column's block max exceeds it by more
        // than kQbSlack (probabilities stay below 2^kQbSlack, exact after the
        // final division), so O is rarely rescaled.
        if (blk == qblk) {
#pragma unroll
            for (int nq = 0; nq < kPfNq; ++nq)
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (tok_base + kt * 16 + 4 * kg + r > pcol[nq]) sacc[nq][kt][r] = -INFINITY;
        }
        bf16x8 pa[kPfNq][4];
#pragma unroll
        for (int nq = 0; nq < kPfNq; ++nq) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[nq][kt][r]);
            mx = max_xor16_32(mx, lane) * scale_log2;
            const bool move = mx > m2[nq] + kQbSlack;
            const float m_new = move ? mx : m2[nq];
            const float alpha = !move ? 1.f : (m2[nq] == -INFINITY ? 0.f : fast_exp2(m2[nq] - m_new));
            const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
            float psum = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float pv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    pv[i] = fast_exp2(fmaf(sacc[nq][2 * c + (i >> 2)][i & 3], scale_log2, neg_m));
                    psum += pv[i];
                }
                const u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                  pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
                pa[nq][c] = as_bf16x8(pk);
            }
            psum = sum_xor16_32(psum, lane);
            lsum[nq] = lsum[nq] * alpha + psum;
            m2[nq] = m_new;
            if (__ballot(move)) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[nq][dt][r] *= alpha;
            }
        }
        // O^T += V^T x P^T (as in pf_attn_kernel, swizzled rows): lane (col, kg)
        // accumulates O[column col][d = dt*16 + 4*kg + r].
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < S / 32; ++c) {
            const int rlo = c * 32 + 4 * kg + (col >> 2);  // rhi = rlo + 16, same swizzle
            const int lp = (col & 3) >> 1, within = (col & 1) * 8;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int off = qb_swz(rlo, dt * 2 + lp) + within;
                const u32x2 lo = lds_read_tr16(v_lds + off);
                const u32x2 hi = lds_read_tr16(v_lds + off + 16 * 256);
                const u32x4 vbv = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int nq = 0; nq < kPfNq; ++nq) o[nq][dt] = mfma16(as_bf16x8(vbv), pa[nq][c], o[nq][dt]);
            }
        }
        // Reads run four d-tiles ahead of the products.
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int i = 0; i < 56; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_barrier(0);
        // The next block has landed (this wave's runs) and every wave is done
        // with this block's buffer.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    }
    // Rows of the call: the normalised output, or zeros / -inf for a row
    // outside the cache.
#pragma unroll
    for (int nq = 0; nq < kPfNq; ++nq) {
        if (trow[nq] < 0) continue;
        const bool has = pcol[nq] >= 0 && lsum[nq] > 0.f;
        const float inv = has ? 1.f / lsum[nq] : 0.f;
        const int64_t hrow = ((int64_t)b * T + trow[nq]) * H + (int64_t)g * R + col % R;
        bf16_t *op = out + hrow * D + 4 * kg;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            *reinterpret_cast<u32x2 *>(op + dt * 16) =
                u32x2{pack_bf16x2(o[nq][dt][0] * inv, o[nq][dt][1] * inv),
                      pack_bf16x2(o[nq][dt][2] * inv, o[nq][dt][3] * inv)};
        if (lse && kg == 0) lse[hrow] = has ? m2[nq] * kLn2 + logf(lsum[nq]) : -INFINITY;
    }
}

// One workgroup per (sequence, row of the pass, group): the kept slots are
// listed once, their (m, l) staged in LDS, then every thread merges four
// d-values of one head over the kept slots. The workgroup is sized to the
// R * D / 4 threads that merge (64 for two heads), so small groups leave no
// idle waves holding the compute units' wave slots.
__global__ __launch_bounds__(256) void pf_merge_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const bf16_t *__restrict__ part_o,
    const float2 *__restrict__ part_ml, int T, int G, int R, int Nmax, int K, int t0, int rows,
    int g0, int ng, bf16_t *__restrict__ out, float *__restrict__ lse) {
    __shared__ int32_t s_sel[KMAX];
    __shared__ int32_t s_kept[KMAX];
    __shared__ int32_t s_n;
    __shared__ float2 s_ml[KMAX * msa::kMaxHeadsPerGroup];
    const int tid = threadIdx.x, lane = tid & 63, nthr = blockDim.x;
    const int64_t unit = blockIdx.x;  // (b, tl, gl), group g0 + gl
    const int g = g0 + (int)(unit % ng);
    const int64_t btl = unit / ng;
    const int b = (int)(btl / rows), tl = (int)(btl % rows);
    const int t = t0 + tl;
    if (t >= T) return;
    const int p = pf_row_pos(kv_lens, q_start, b, t, T, Nmax);
    if (tid < K) s_sel[tid] = p >= 0 ? sel[(((int64_t)b * T + t) * G + g) * K + tid] : -1;
    __syncthreads();
    if (tid < 64) {  // K <= KMAX = 64: one wave lists the kept slots
        const bool keep = lane < K && p >= 0 && slot_kept(s_sel, lane, p / S + 1);
        const uint64_t m = __ballot(keep);
        if (keep) s_kept[__popcll(m & ((1ull << lane) - 1ull))] = lane;
        if (lane == 0) s_n = __popcll(m);
    }
    __syncthreads();
    const int n = s_n;
    const int64_t slot0 = unit * K;
    for (int i = tid; i < n * R; i += nthr) s_ml[i] = part_ml[(slot0 + s_kept[i / R]) * R + i % R];
    __syncthreads();
    const int H = G * R;
    for (int idx = tid; idx < R * (D / 4); idx += nthr) {
        const int r = idx / (D / 4), d0 = (idx % (D / 4)) * 4;
        float M = -INFINITY;
        for (int i = 0; i < n; ++i) M = fmaxf(M, s_ml[i * R + r].x);
        float L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int i = 0; i < n; ++i) {
            const float2 ml = s_ml[i * R + r];
            const float wk = fast_exp2(ml.x - M) * ml.y;
            L += wk;
            const u32x2 ov =
                *reinterpret_cast<const u32x2 *>(part_o + ((slot0 + s_kept[i]) * R + r) * D + d0);
            acc[0] += wk * __uint_as_float(ov[0] << 16);
            acc[1] += wk * __uint_as_float(ov[0] & 0xFFFF0000u);
            acc[2] += wk * __uint_as_float(ov[1] << 16);
            acc[3] += wk * __uint_as_float(ov[1] & 0xFFFF0000u);
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        bf16_t *op = out + (((int64_t)b * T + t) * H + (int64_t)g * R + r) * D + d0;
        *reinterpret_cast<u32x2 *>(op) =
            u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        if (lse && d0 == 0)
            lse[((int64_t)b * T + t) * H + (int64_t)g * R + r] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
    }
}

}  // namespace

namespace msa {

// The list build of one pass (rows t0 .. t0 + rows - 1, groups g0 .. g0 + ng - 1).
void build_pass_lists(const PrefillWs &w, char *base, const int32_t *sel,
                      const int32_t *kv_lens, const int32_t *q_start, int B, int T, int G,
                      int Nmax, int K, int t0, int g0, hipStream_t st) {
    const int ng = w.groups;
    const int W = w.bit_words;
    uint32_t *bits = reinterpret_cast<uint32_t *>(base + w.bits_off);
    int32_t *wpre = reinterpret_cast<int32_t *>(base + w.wpre_off);
    int32_t *counts = reinterpret_cast<int32_t *>(base + w.counts_off);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + w.offsets_off);
    int32_t *tile_first = reinterpret_cast<int32_t *>(base + w.tile_first_off);
    int32_t *tile_map = reinterpret_cast<int32_t *>(base + w.tile_map_off);
    int32_t *list = reinterpret_cast<int32_t *>(base + w.list_off);
    const unsigned slot_blocks = (unsigned)((w.nslots + 255) / 256);
    const int wchunks = (W + 1023) / 1024;
    const int write_all = w.nb_max <= kPfMarkAllBlocks;
    if (!write_all)
        pf_clear_kernel<<<(unsigned)(w.nlists * wchunks), 256, 0, st>>>(bits, kv_lens, W, wchunks,
                                                                        ng, w.nb_max, Nmax);
    if (w.nb_max <= kPfMarkLdsBlocks)
        pf_mark_lds_kernel<<<(unsigned)((int64_t)B * W * ng), 256,
                             (size_t)(w.nb_max + 32 * K) * 4, st>>>(
            sel, kv_lens, q_start, T, G, Nmax, K, t0, w.rows, g0, ng, w.nb_max, W, write_all,
            bits);
    else
        pf_mark_kernel<<<slot_blocks, 256, 0, st>>>(sel, kv_lens, q_start, B, T, G, Nmax, K, t0,
                                                    w.rows, g0, ng, w.nb_max, W, bits);
    pf_rank_kernel<<<(unsigned)((w.nlists + 3) / 4), 256, 0, st>>>(bits, w.nlists, W, kv_lens, ng,
                                                                   w.nb_max, Nmax, wpre, counts);
    if (w.nlists <= kScanSmall)
        pf_scan_small_kernel<<<1, 1024, 0, st>>>(counts, w.nlists, w.entries_per_tile, offsets,
                                                 tile_first, tile_map);
    else
        pf_scan_kernel<<<1, 1024, 0, st>>>(counts, w.nlists, w.entries_per_tile, offsets,
                                           tile_first, tile_map);
    if (w.nb_max <= kPfMarkLdsBlocks)
        pf_scatter_lds_kernel<<<(unsigned)((int64_t)B * W * ng), 256,
                                (size_t)(w.nb_max + 32 * K) * 4, st>>>(
            sel, kv_lens, q_start, wpre, offsets, T, G, Nmax, K, t0, w.rows, g0, ng, w.nb_max, W,
            list);
    else
        pf_scatter_kernel<<<slot_blocks, 256, 0, st>>>(sel, kv_lens, q_start, bits, wpre, offsets,
                                                       B, T, G, Nmax, K, t0, w.rows, g0, ng,
                                                       w.nb_max, W, list);
}

// Pooled block scores of T*G > kScanMaxRows rows: the MFMA prefill index
// kernel without the top-K epilogue.
constexpr int64_t kIdxSplitWgs = 512;
msa_status launch_prefill_pooled(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                 const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                                 const int32_t *q_start, float *pooled, int64_t nb_max,
                                 hipStream_t st) {
    const int G = cfg->num_kv_groups;
    const int rows = T * G;
    const bool f8 = cfg->index_dtype == MSA_FP8_E4M3;
    const unsigned char *qi = static_cast<const unsigned char *>(q_idx);
    const unsigned char *ki = static_cast<const unsigned char *>(k_idx);
    // A short prefill's few row tiles split their key blocks over up to
    // kIdxSplitWgs workgroups in all.
    const int64_t tiles = ((int64_t)rows + kPfRows - 1) / kPfRows * B;
    const int64_t nz = tiles >= kIdxSplitWgs ? 1 : min(kIdxSplitWgs / tiles, nb_max);
    const int bps = (int)((nb_max + nz - 1) / nz);
    const int nzb = (int)((nb_max + bps - 1) / bps);
    const dim3 grid((unsigned)((rows + kPfRows - 1) / kPfRows), (unsigned)B, (unsigned)nzb);
    if (f8)
        idx_prefill_kernel<true, 0><<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G,
                                                          Nmax, nb_max, 0, nullptr, nullptr, 0,
                                                          nzb > 1 ? bps : 0);
    else
        idx_prefill_kernel<false, 0><<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G,
                                                           Nmax, nb_max, 0, nullptr, nullptr, 0,
                                                           nzb > 1 ? bps : 0);
    return launch_status("prefill index kernel");
}


}  // namespace msa

extern "C" {

msa_status msa_index_topk(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                          const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                          const int32_t *q_start, int32_t *sel, float *sel_scores,
                          void *workspace, size_t ws_bytes, void *stream) {
    msa::clear_error();
    msa_status s = msa::check_index_args(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, sel,
                                         sel_scores, workspace, ws_bytes);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int G = cfg->num_kv_groups, K = cfg->topk;
    if (!msa::index_uses_pooled(cfg, B, T)) {
        // Prefill: scores, block max and the row's top-K in one kernel.
        const bool f8 = cfg->index_dtype == MSA_FP8_E4M3;
        const unsigned char *qi = static_cast<const unsigned char *>(q_idx);
        const unsigned char *ki = static_cast<const unsigned char *>(k_idx);
        const int64_t nbm = ((int64_t)Nmax + S - 1) / S;
        const dim3 grid((unsigned)(((int64_t)T * G + kPfRows - 1) / kPfRows), (unsigned)B);
#define MSA_IDX_PREFILL(F8_, KC_)                                                              \
    idx_prefill_kernel<F8_, KC_><<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, nullptr, T, G, \
                                                       Nmax, nbm, K, sel, sel_scores)
        if (f8 && K <= 16) MSA_IDX_PREFILL(true, 16);
        else if (f8) MSA_IDX_PREFILL(true, 32);
        else if (K <= 16) MSA_IDX_PREFILL(false, 16);
        else MSA_IDX_PREFILL(false, 32);
#undef MSA_IDX_PREFILL
        return launch_status("prefill index kernel");
    }
    // Decode shapes, K above the register top-K and short prefills: pooled
    // scores into the workspace, then a wavefront ranks each row.
    return msa::launch_scan_topk(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, sel, sel_scores,
                                 workspace, st);
}

msa_status msa_index_pool(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                          const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                          const int32_t *q_start, float *pooled, void *stream) {
    msa::clear_error();
    msa_status s =
        msa::check_pool_args(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, pooled);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    return msa::launch_pooled(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, pooled,
                         ((int64_t)Nmax + S - 1) / S, reinterpret_cast<hipStream_t>(stream));
}

msa_status msa_sparse_attn_prefill(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                   const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *kv_lens, const int32_t *q_start,
                                   const int32_t *sel, void *out, float *lse, void *workspace,
                                   size_t ws_bytes, void *stream) {
    msa::clear_error();
    msa_status s = msa::check_sparse_args(cfg, B, T, Nmax, q, k_cache, v_cache, kv_lens, q_start,
                                          sel, out, lse, workspace, ws_bytes,
                                          MSA_WS_SPARSE_PREFILL);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int G = cfg->num_kv_groups, R = cfg->heads_per_group, K = cfg->topk;
    const float sl2 = scale_log2_of(cfg);
    const bf16_t *qp = static_cast<const bf16_t *>(q);
    const bf16_t *kp = static_cast<const bf16_t *>(k_cache);
    const bf16_t *vp = static_cast<const bf16_t *>(v_cache);
    bf16_t *op = static_cast<bf16_t *>(out);
    const msa::PrefillWs w = msa::prefill_ws(cfg, B, T, Nmax);
    if (!w.kv_major) {
        const int64_t units = (int64_t)B * T * G;
        sparse_attn_kernel<<<(unsigned)units, 256, 0, st>>>(qp, kp, vp, kv_lens, q_start, sel, T,
                                                           G, R, Nmax, K, sl2, op, lse);
        return launch_status("sparse attention kernel");
    }
    char *base = static_cast<char *>(workspace);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + w.offsets_off);
    int32_t *tile_first = reinterpret_cast<int32_t *>(base + w.tile_first_off);
    int32_t *tile_map = reinterpret_cast<int32_t *>(base + w.tile_map_off);
    int32_t *list = reinterpret_cast<int32_t *>(base + w.list_off);
    bf16_t *part_o = reinterpret_cast<bf16_t *>(base + w.part_o_off);
    float2 *part_ml = reinterpret_cast<float2 *>(base + w.part_ml_off);
    // Merge threads: R * D / 4 rounded up to whole waves, at most 256 (K <= 64
    // needs one wave, which every size here has).
    const unsigned merge_threads = (unsigned)std::min(256, (R * (D / 4) + 63) / 64 * 64);
    for (int32_t g0 = 0; g0 < G; g0 += w.groups)
      for (int32_t t0 = 0; t0 < T; t0 += w.rows) {
        const int ng = w.groups;
        msa::build_pass_lists(w, base, sel, kv_lens, q_start, B, T, G, Nmax, K, t0, g0, st);
        pf_attn_kernel<<<(unsigned)w.max_tiles, 256, 0, st>>>(
            qp, kp, vp, kv_lens, q_start, offsets, tile_first, tile_map, list, w.nlists, T, G, R,
            Nmax, K, t0, w.rows, g0, ng, w.nb_max, w.entries_per_tile, sl2, part_o, part_ml,
            reinterpret_cast<unsigned char *>(base + w.trash_off));
        pf_merge_kernel<<<(unsigned)((int64_t)B * w.rows * ng), merge_threads, 0, st>>>(
            sel, kv_lens, q_start, part_o, part_ml, T, G, R, Nmax, K, t0, w.rows, g0, ng, op, lse);
        s = launch_status("sparse prefill kernels");
        if (s != MSA_OK) return s;
    }
    return MSA_OK;
}

msa_status msa_index_topk_qblock(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                 const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                                 const int32_t *q_start, int32_t *sel, float *sel_scores,
                                 void *stream) {
    msa::clear_error();
    msa_status s = msa::check_qblock_index_args(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start,
                                                sel, sel_scores);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int G = cfg->num_kv_groups, K = cfg->topk;
    const int nslots = msa::qblock_slots(T);
    const bool f8 = cfg->index_dtype == MSA_FP8_E4M3;
    const unsigned char *qi = static_cast<const unsigned char *>(q_idx);
    const unsigned char *ki = static_cast<const unsigned char *>(k_idx);
    const int64_t nbm = ((int64_t)Nmax + S - 1) / S;
    const dim3 grid((unsigned)((int64_t)nslots * ((G + 1) / 2)), (unsigned)B);
#define MSA_IDX_QBLOCK(F8_, KC_)                                                                 \
    idx_prefill_kernel<F8_, KC_, true><<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, nullptr, \
                                                             T, G, Nmax, nbm, K, sel,           \
                                                             sel_scores, nslots)
    if (f8 && K <= 16) MSA_IDX_QBLOCK(true, 16);
    else if (f8) MSA_IDX_QBLOCK(true, 32);
    else if (K <= 16) MSA_IDX_QBLOCK(false, 16);
    else MSA_IDX_QBLOCK(false, 32);
#undef MSA_IDX_QBLOCK
    return launch_status("query-block index kernel");
}

msa_status msa_sparse_attn_prefill_qblock(const msa_config *cfg, int32_t B, int32_t T,
                                          int32_t Nmax, const void *q, const void *k_cache,
                                          const void *v_cache, const int32_t *kv_lens,
                                          const int32_t *q_start, const int32_t *sel, void *out,
                                          float *lse, void *stream) {
    msa::clear_error();
    msa_status s = msa::check_sparse_args(cfg, B, T, Nmax, q, k_cache, v_cache, kv_lens, q_start,
                                          sel, out, lse, nullptr, 0, -1);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    const int G = cfg->num_kv_groups, R = cfg->heads_per_group, K = cfg->topk;
    const int nslots = msa::qblock_slots(T);
    const int ppw = kQbWaves * kPfNq * (16 / R);
    const int ncw = (S + ppw - 1) / ppw;
    const int64_t nunits = (int64_t)B * nslots * G;
    const int64_t nwg = (nunits + 7) / 8 * 8 * ncw;
    if (nwg > 0x7FFFFFFF)
        return msa::fail(MSA_ERR_UNSUPPORTED, "too many query blocks for one launch");
    qb_attn_kernel<<<(unsigned)nwg, kQbWaves * 64, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k_cache),
        static_cast<const bf16_t *>(v_cache), kv_lens, q_start, sel, T, G, R, Nmax, K, nslots,
        ncw, nunits, scale_log2_of(cfg), static_cast<bf16_t *>(out), lse);
    return launch_status("query-block sparse attention kernel");
}

msa_status msa_cache_append(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                            const void *k_new, const void *v_new, const void *k_idx_new,
                            const int32_t *pos0, void *k_cache, void *v_cache, void *k_idx,
                            void *stream) {
    msa::clear_error();
    msa_status s = msa::check_append_args(cfg, B, T, Nmax, k_new, v_new, k_idx_new, pos0,
                                          k_cache, v_cache, k_idx);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    const int64_t rows = (int64_t)B * T;
    const int kib = DI * (cfg->index_dtype == MSA_FP8_E4M3 ? 1 : 2);
    cache_append_kernel<<<(unsigned)((rows + 3) / 4), 256, 0,
                          reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4 *>(k_new), static_cast<const u32x4 *>(v_new),
        static_cast<const unsigned char *>(k_idx_new), pos0, B, T, cfg->num_kv_groups, Nmax, kib,
        static_cast<u32x4 *>(k_cache), static_cast<u32x4 *>(v_cache),
        static_cast<unsigned char *>(k_idx));
    return launch_status("cache append kernel");
}

}  // extern "C"

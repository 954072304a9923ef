// libmsa decode kernels for gfx950 (MI355X, CDNA4) and the decode entry points.
//
// The method (MiniMax M3 sparse attention, cloud.tencent.com article
// "Something BIG Is Coming 百万token上下文提速近10倍，MiniMax M3的稀疏注意力凭什么这么快"):
// §二 an index query per GQA group scores the KV blocks (block max-pool of
// per-token scores) and keeps the top-k blocks; full softmax attention runs
// over only those blocks; §六 all heads of a group share them. At decode the
// index keys are the dominant stream (the pages' decode is memory-bound).
//
// Kernels:
//   idx_scan_kernel      decode index scores: streams k_idx once for all
//                        groups through LDS, 16x16x32 bf16 (or 16x16x128
//                        E4M3) MFMA, causal block max in registers; writes
//                        pooled scores.
//   topk_rows_kernel     one wavefront per row: a bitonic sort of the lanes'
//                        best scores sets a threshold, the candidates above it
//                        are compacted and one bitonic sort of 64-bit keys
//                        (score, inverted block id) across lanes ranks them.
//   sparse_decode_kernel one workgroup of 8 or 16 waves per (sequence, group,
//                        split), one 32-token chunk per wave; optionally
//                        ranks the row's blocks itself; waves merge in LDS
//                        into a partial per split; with arrival counters
//                        (msa_decode) the last split of a (sequence, group)
//                        merges them all.
//   combine_kernel       (msa_sparse_attn_decode) log-sum-exp merge of the
//                        split partials.
#include "msa_device.h"

namespace {

// ---------------------------------------------------------------------------
// Decode index scores (T*G <= 16 rows per sequence).
//
// Every index key of the sequence is streamed once and serves all T*G
// index-query rows. Workgroup x of sequence y takes blocks_per_wg blocks;
// each wave walks its blocks in steps of 16 KiB of keys (64 bf16 or 128 fp8
// tokens): a step is read with sixteen load instructions of one contiguous KiB
// each and staged in the wave's own LDS region (rows padded by 16 bytes),
// while the loads of the next step are already in flight. The MFMA
// D = A x B then takes A = index-query rows (16 rows, m = t*G + g, zero above
// T*G) from registers and B = k_idx^T for 16 tokens from LDS; output lane l
// holds D[4*(l>>4) + r][l & 15], i.e. rows 4*(l>>4)..+3 of one token. A
// running per-row max over the block's tiles, then a 16-lane max, gives the
// block's pooled score, written to pooled[b][m][block].
//
// bf16 keys use four 16x16x32 bf16 MFMAs per 16-token tile; OCP E4M3 keys one
// 16x16x128 f8f6f4 MFMA (unit scales). Index data are small integers in
// practice, so both sums are exact in fp32.
// MI355X's last-level (Infinity) cache, 256 MiB.
constexpr int64_t kLastLevelCacheBytes = 256ll << 20;

// A split partial word that this call has not written yet (msa_decode): a
// NaN pattern the arithmetic never produces (hardware NaNs are the canonical
// quiet NaN or carry a bf16 input's payload, whose low 16 bits are zero).
constexpr uint32_t kUnpublished = 0xFFFFFFFFu;
// Bound of the wait for a partial word (each wait sleeps 64 clocks): the
// words are stored before their split's arrival is counted, so the wait ends
// at once in practice; the bound keeps every wave's exit guaranteed.
constexpr int kPublishSpin = 1 << 20;

template <bool F8>
struct ScanGeom {
    static constexpr int kRowBytes = DI * (F8 ? 1 : 2);     // one token's key
    static constexpr int kRow = kRowBytes + 16;              // LDS row stride
    static constexpr int kStep = F8 ? 128 : 64;              // tokens per step
    static constexpr int kLanesPerRow = kRowBytes / 16;
    static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
    static constexpr int kLoads = kStep / kRowsPerLoad;      // 16
    static constexpr int kStepsPerBlock = S / kStep;
    static constexpr int kWaveLds = kStep * kRow;
};

template <bool F8, bool Stream>
__global__ __launch_bounds__(256) void idx_scan_kernel(
    const unsigned char *__restrict__ q_idx, const unsigned char *__restrict__ k_idx,
    const int32_t *__restrict__ kv_lens, const int32_t *__restrict__ q_start,
    float *__restrict__ pooled, int T, int G, int Nmax, int64_t nb_max, int blocks_per_wg,
    int32_t *__restrict__ zero_counters, uint32_t *__restrict__ unpublish, int64_t n_unpublish) {
    typedef ScanGeom<F8> Geo;
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * Geo::kWaveLds];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Reset the decode attention kernel's state of the same call (msa_decode):
    // zero its arrival counters (one per (sequence, group)) and mark every
    // word of its split partials unpublished, each workgroup a slice; the
    // kernel boundary orders these stores before that kernel.
    if (zero_counters && blockIdx.x == 0)
        for (int i = threadIdx.x; i < G; i += 256) zero_counters[(int64_t)b * G + i] = 0;
    if (unpublish) {
        const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
        const int64_t per = (n_unpublish + nwg - 1) / nwg;
        const int64_t lo = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * per;
        const int64_t hi = min(lo + per, n_unpublish);
        // Agent-scope (write-through) stores: plain ones would be left dirty
        // in the L2 for the end-of-kernel write-back (measured slower).
        for (int64_t i = lo + threadIdx.x; i < hi; i += 256)
            __hip_atomic_store(&unpublish[i], kUnpublished, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    const int rows = T * G;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int p_hi = min(qs + T - 1, kv - 1);
    if (p_hi < 0) return;
    const int nb = p_hi / S + 1;
    const int blk_begin = blockIdx.x * blocks_per_wg;
    const int blk_end = min(blk_begin + blocks_per_wg, nb);
    const int my_blocks = blk_begin + wave < blk_end ? (blk_end - blk_begin - wave + 3) / 4 : 0;
    const int nsteps = my_blocks * Geo::kStepsPerBlock;
    if (nsteps == 0) return;

    const int col = lane & 15, kg = lane >> 4;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    // A operand: index-query row `col`, key bytes [kg*32, kg*32+32) of every
    // 128-byte K slice (bf16: four slices of 32 elements; fp8: one slice).
    u32x4 a[4][2];
    {
        const unsigned char *qp =
            q_idx + ((size_t)b * rows + (col < rows ? col : 0)) * Geo::kRowBytes;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            if (F8 && kc > 0) break;
            const int off = F8 ? kg * 32 : kc * 64 + kg * 16;
            a[kc][0] = col < rows ? ld16(qp + off) : zero4;
            a[kc][1] = (F8 && col < rows) ? ld16(qp + off + 16) : zero4;
        }
    }
    int prow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kg + r;
        const int p = qs + m / G;
        prow[r] = (m < rows && p >= 0 && p < kv) ? p : -1;
    }
    const unsigned char *kbytes = k_idx + (size_t)b * Nmax * Geo::kRowBytes;
    unsigned char *my = lds + wave * Geo::kWaveLds;
    // Step s covers tokens [tok, tok + kStep) of block blk_begin + wave + 4*(s / steps per block).
    auto step_tok = [&](int s) {
        return (blk_begin + wave + 4 * (s / Geo::kStepsPerBlock)) * S +
               (s % Geo::kStepsPerBlock) * Geo::kStep;
    };
    const int lrow = lane / Geo::kLanesPerRow, lcol = (lane % Geo::kLanesPerRow) * 16;
    u32x4 v[Geo::kLoads];
    auto load_step = [&](int s) {
        const int t0 = step_tok(s);
#pragma unroll
        for (int i = 0; i < Geo::kLoads; ++i) {
            const int tok = t0 + Geo::kRowsPerLoad * i + lrow;
            const unsigned char *src = kbytes + (size_t)tok * Geo::kRowBytes + lcol;
            v[i] = tok < kv ? (Stream ? ld16_stream(src) : ld16(src)) : zero4;
        }
    };
    load_step(0);
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int s = 0; s < nsteps; ++s) {
        const int t0 = step_tok(s);
#pragma unroll
        for (int i = 0; i < Geo::kLoads; ++i)
            *reinterpret_cast<u32x4 *>(my + (Geo::kRowsPerLoad * i + lrow) * Geo::kRow + lcol) = v[i];
        if (s + 1 < nsteps) load_step(s + 1);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's LDS rows have landed
        __builtin_amdgcn_wave_barrier();
        const bool need_mask = t0 + Geo::kStep - 1 > qs;
#pragma unroll
        for (int tile = 0; tile < Geo::kStep / 16; ++tile) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const unsigned char *brow = my + (tile * 16 + col) * Geo::kRow;
            if constexpr (F8) {
                const u32x4 b0 = *reinterpret_cast<const u32x4 *>(brow + kg * 32);
                const u32x4 b1 = *reinterpret_cast<const u32x4 *>(brow + kg * 32 + 16);
                acc = mfma16_f8(cat_i32x8(a[0][0], a[0][1]), cat_i32x8(b0, b1), acc);
            } else {
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    acc = mfma16(as_bf16x8(a[kc][0]),
                                 as_bf16x8(*reinterpret_cast<const u32x4 *>(brow + kc * 64 + kg * 16)),
                                 acc);
            }
            const int tok = t0 + tile * 16 + col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sc = (need_mask && tok > prow[r]) ? -INFINITY : acc[r];
                mx[r] = fmaxf(mx[r], sc);
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (s % Geo::kStepsPerBlock == Geo::kStepsPerBlock - 1) {  // block complete
            const int blk = t0 / S;
            float m2[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                m2[r] = mx[r];
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) m2[r] = fmaxf(m2[r], __shfl_xor(m2[r], off));
                mx[r] = -INFINITY;
            }
            if (col == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (prow[r] >= blk * S)
                        pooled[((size_t)b * rows + 4 * kg + r) * nb_max + blk] = m2[r] + 0.0f;
            }
        }
    }
}

// Top-K of rows (b, t, g) from their pooled scores: one wavefront per row,
// four rows per workgroup. Rows outside the cache get -1.
__global__ __launch_bounds__(256) void topk_rows_kernel(
    const float *__restrict__ pooled, int64_t nb_max, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, int B, int T, int G, int Nmax, int K,
    int32_t *__restrict__ sel, float *__restrict__ sel_scores) {
    __shared__ uint64_t s_buf[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    const int rows = T * G;
    if (row >= (int64_t)B * rows) return;
    const int b = (int)(row / rows);
    const int t = (int)(row % rows) / G;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int p = qs + t;
    uint64_t top = 0;
    if (p >= 0 && p < kv)
        top = wave_topk_row_short(pooled + row * nb_max, p / S + 1, p / S + 1, K, lane,
                                  s_buf[wave]);
    if (lane < K) {
        sel[row * K + lane] = top ? key_block(top) : -1;
        if (sel_scores) sel_scores[row * K + lane] = top ? key_score(top) : -INFINITY;
    }
}

// The value of split partial word *p once its split has stored it: v is a
// first agent-scope read of it; re-read (bounded) while it is still the
// kUnpublished mark of this call.
__device__ __forceinline__ float published(const float *p, float v) {
    for (int spin = 0; __float_as_uint(v) == kUnpublished && spin < kPublishSpin; ++spin) {
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return v;
}

// Decode: the new token of sequence b sits at position kv - 1. Group g's
// kept blocks give 4*nblk 32-token chunks; workgroup (b, g, split) has NW
// waves (16 when the grid fills the GPU, else 8; msa::decode_waves) and
// takes chunks [NW*split, NW*split + NW), one per wave, so every load of the
// split is in flight at once (with 16 waves one workgroup fills a CU's LDS:
// the V staging takes 144 KiB). With `pooled` non-null each workgroup first
// ranks the row itself (rows of up to kShortRow blocks by wave 0, longer
// ones by all waves; split 0 also writes sel / sel_scores), otherwise it
// reads sel. The waves merge in LDS into one unnormalised partial (O, m, l)
// per split, which combine_kernel merges by log-sum-exp (or, in msa_decode,
// the last split of (b, g) to finish).
constexpr int kShortRow = 1024;

template <int NW>
struct DecodeLds {
    // Ranking: the waves' candidate lists and sorted runs (2 x NW x 64 keys);
    // then the waves' V chunks; then [NW][16][128] fp32 outputs (the waves'
    // merge).
    __attribute__((aligned(16))) unsigned char vrows[NW * kVWave];
    int sel[KMAX];
    int blocks[KMAX];
    int nblk;
    float m[NW * 16], l[NW * 16];
    float sc[NW * 16];     // each wave's weight per head
    float hm[16], hl[16];  // per head: max of the waves' m, weighted sum of l
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_decode_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache,
    const bf16_t *__restrict__ v_cache, const int32_t *__restrict__ kv_lens,
    const float *__restrict__ pooled, int64_t nb_max, int32_t *__restrict__ sel,
    float *__restrict__ sel_scores, int G, int R, int Nmax, int K, int nsplit, float scale_log2,
    float *__restrict__ part_o, float *__restrict__ part_ml, int32_t *__restrict__ counters,
    bf16_t *__restrict__ out, float *__restrict__ lse) {
    __shared__ DecodeLds<NW> L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = (int)(blockIdx.x % nsplit);
    const int64_t unit = blockIdx.x / nsplit;  // (sequence, group)
    const int g = (int)(unit % G);
    const int b = (int)(unit / G);
    const int H = G * R;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int p = kv - 1;
    // The query does not depend on the selection: its loads overlap the ranking.
    bf16x8 qf[4];
    load_query(qf, q + ((int64_t)b * H + (int64_t)g * R) * D, R, lane);
    if (pooled) {
        // Every split ranks the row alike (a wave's ranking is shorter than
        // publishing one split's to the others): wave 0 alone up to kShortRow
        // blocks, else every wave a share and wave 0 merges their runs.
        // n_load = nb_max: the row's pooled scores are loaded while kv_lens is
        // still in flight.
        uint64_t *kbuf = reinterpret_cast<uint64_t *>(L.vrows);
        const float *row = pooled + unit * nb_max;
        const int n = p >= 0 ? p / S + 1 : 0;
        uint64_t top = 0;
        if (nb_max <= kShortRow) {
            if (wave == 0) top = wave_topk_row_short(row, n, (int)nb_max, K, lane, kbuf);
        } else {
            top = block_topk_row<NW>(row, n, (int)nb_max, K, lane, wave, kbuf, kbuf + NW * 64);
        }
        if (wave == 0) {
            if (lane < K) {
                const int blk = top ? key_block(top) : -1;
                L.sel[lane] = blk;
                if (split == 0) {
                    sel[unit * K + lane] = blk;
                    if (sel_scores) sel_scores[unit * K + lane] = top ? key_score(top) : -INFINITY;
                }
            }
        }
    } else if (tid < K) {
        L.sel[tid] = p >= 0 ? sel[unit * K + tid] : -1;
    }
    __syncthreads();
    if (wave == 0) {
        const int n = build_block_list(L.sel, K, p, L.blocks, lane, pooled != nullptr);
        if (lane == 0) L.nblk = n;
    }
    __syncthreads();
    const int c = split * NW + wave;  // this wave's chunk
    WaveAttn st;
    wave_attn_init(st);
    if (c < L.nblk * 4) {
        // Each kept chunk is read by this wave alone: streaming loads.
        attend_chunk<true>(st, qf, k_cache + ((size_t)b * G + g) * Nmax * D,
                     v_cache + ((size_t)b * G + g) * Nmax * D, L.blocks[c >> 2] * S + (c & 3) * 32,
                     p, scale_log2, L.vrows + wave * kVWave, lane);
    }
    // Merge the NW waves into this split's partial: per head h the max M of
    // the waves' m, each wave's weight exp2(m_w - M) and the weighted sum L of
    // their l are computed once, by one thread per (wave, head); each wave then
    // writes its O scaled by its weight, and every thread sums one (head, d)
    // element over the waves.
    float *s_o = reinterpret_cast<float *>(L.vrows);
    const int col = lane & 15, kg = lane >> 4;
    if (lane < 16) {
        L.m[wave * 16 + lane] = st.m;
        L.l[wave * 16 + lane] = st.l;
    }
    __syncthreads();
    if (tid < NW * 16 && (tid & 15) < R) {
        const int w0 = tid >> 4, h = tid & 15;
        float mv[NW];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mv[w] = L.m[w * 16 + h];
            M = fmaxf(M, mv[w]);
        }
        L.sc[tid] = mv[w0] == -INFINITY ? 0.f : exp2f(mv[w0] - M);
        if (w0 == 0) {
            float Lsum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if (mv[w] != -INFINITY) Lsum += exp2f(mv[w] - M) * L.l[w * 16 + h];
            L.hm[h] = M;
            L.hl[h] = Lsum;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * kg + r;
        if (h >= R) continue;
        const float sc = L.sc[wave * 16 + h];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) s_o[(wave * 16 + h) * D + dt * 16 + col] = st.o[dt][r] * sc;
    }
    __syncthreads();
    for (int idx = tid; idx < R * D; idx += NW * 64) {
        const int h = idx / D, dd = idx % D;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += s_o[(w * 16 + h) * D + dd];
        const float M = L.hm[h], Lsum = L.hl[h];
        const int64_t pu = (unit * nsplit + split) * R + h;
        if (counters) {
            // Agent-scope stores (written through the XCD's L2): the merging
            // workgroup may run on another XCD, behind another L2.
            __hip_atomic_store(&part_o[pu * D + dd], acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (dd == 0) {
                __hip_atomic_store(&part_ml[pu * 2], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&part_ml[pu * 2 + 1], Lsum, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            part_o[pu * D + dd] = acc;
            if (dd == 0) {
                part_ml[pu * 2] = M;
                part_ml[pu * 2 + 1] = Lsum;
            }
        }
    }
    if (!counters) return;
    // The last of the nsplit workgroups of (sequence, group) to arrive merges
    // all partials. No fence orders the partials before the arrival (an
    // agent-scope release writes back the whole L2 and costs more than the
    // merge): instead every partial word is an agent-scope atomic that this
    // call writes exactly once, over the kUnpublished value the index kernel
    // of the same call stored, and the merging workgroup reads each word until
    // it holds its split's value. Coherence of a single atomic location makes
    // that value the one the split stored; the arrival counter only chooses
    // the merging workgroup, so it is counted while the partial stores are
    // still on their way (the merging workgroup's reads wait for them).
    __syncthreads();
    if (tid == 0)
        L.nblk = __hip_atomic_fetch_add(&counters[unit], 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
    __syncthreads();
    if (!L.nblk) return;
    // One round of loads per batch of eight splits, merged online.
    for (int idx = tid; idx < R * D; idx += NW * 64) {
        const int h = idx / D, dd = idx % D;
        const int64_t pu0 = unit * nsplit * R + h;
        float M = -INFINITY, Lsum = 0.f, acc = 0.f;
        for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
            float pm[8], pl[8], pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t pu = pu0 + (int64_t)min(sp0 + j, nsplit - 1) * R;
                pm[j] = __hip_atomic_load(&part_ml[pu * 2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                pl[j] = __hip_atomic_load(&part_ml[pu * 2 + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                pv[j] = __hip_atomic_load(&part_o[pu * D + dd], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t pu = pu0 + (int64_t)min(sp0 + j, nsplit - 1) * R;
                pm[j] = published(&part_ml[pu * 2], pm[j]);
                pl[j] = published(&part_ml[pu * 2 + 1], pl[j]);
                pv[j] = published(&part_o[pu * D + dd], pv[j]);
                if (sp0 + j >= nsplit) pm[j] = -INFINITY;
            }
            float Mb = M;
#pragma unroll
            for (int j = 0; j < 8; ++j) Mb = fmaxf(Mb, pm[j]);
            if (Mb == -INFINITY) continue;
            const float sc = M == -INFINITY ? 0.f : exp2f(M - Mb);
            Lsum *= sc;
            acc *= sc;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (pm[j] == -INFINITY) continue;
                const float w = exp2f(pm[j] - Mb);
                Lsum += w * pl[j];
                acc += w * pv[j];
            }
            M = Mb;
        }
        const int64_t uh = unit * R + h;
        out[uh * D + dd] = to_bf16(Lsum > 0.f ? acc / Lsum : 0.f);
        if (lse && dd == 0) lse[uh] = Lsum > 0.f ? M * kLn2 + logf(Lsum) : -INFINITY;
    }
}

// Log-sum-exp merge of the nsplit partials of one (sequence, group, head):
// one thread per output element, every split's partial row read coalesced.
__global__ __launch_bounds__(128) void combine_kernel(const float *__restrict__ part_o,
                                                      const float *__restrict__ part_ml, int G,
                                                      int R, int nsplit, bf16_t *__restrict__ out,
                                                      float *__restrict__ lse) {
    const int64_t uh = blockIdx.x;  // (sequence * G + g) * R + h
    const int h = (int)(uh % R);
    const int64_t unit = uh / R;
    const int dd = threadIdx.x;
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, part_ml[((unit * nsplit + sp) * R + h) * 2]);
    float Lsum = 0.f, acc = 0.f;
    if (M != -INFINITY) {
        for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
            float pv[8], pm[8], pl[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool ok = sp0 + j < nsplit;
                const int64_t pu = (unit * nsplit + sp0 + j) * R + h;
                pv[j] = ok ? part_o[pu * D + dd] : 0.f;
                pm[j] = ok ? part_ml[pu * 2] : -INFINITY;
                pl[j] = ok ? part_ml[pu * 2 + 1] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (pm[j] == -INFINITY) continue;
                const float w = exp2f(pm[j] - M);
                Lsum += w * pl[j];
                acc += w * pv[j];
            }
        }
    }
    // out / lse rows of (sequence, group) are contiguous over the R heads.
    out[uh * D + dd] = to_bf16(Lsum > 0.f ? acc / Lsum : 0.f);
    if (lse && dd == 0) lse[uh] = Lsum > 0.f ? M * kLn2 + logf(Lsum) : -INFINITY;
}

// Sets n words to v (the decode attention state when the MFMA index kernel,
// which does not reset it, produces the pooled scores).
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *__restrict__ p, int64_t n,
                                                       uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// Blocks per decode-scan workgroup: four, one per wave (measured best on the
// 16 x 131072 decode, and on the 4 x 1048576 one: 157 us against 163 us with
// eight, where the grid had been capped near 4096 workgroups).
int64_t scan_blocks_per_wg(int32_t B, int64_t nb_max) {
    (void)B;
    (void)nb_max;
    return 4;
}

// Split partials of msa_sparse_attn_decode and msa_decode: sparse_decode_kernel
// for every (sequence, group, split), then the merge.
static msa_status launch_decode_attention(const msa_config *cfg, int32_t B, int32_t Nmax,
                                          const void *q, const void *k_cache,
                                          const void *v_cache, const int32_t *kv_lens,
                                          const float *pooled, int64_t nb_max, int32_t *sel,
                                          float *sel_scores, void *out, float *lse,
                                          float *part_o, float *part_ml, hipStream_t st,
                                          int32_t *counters = nullptr) {
    const int G = cfg->num_kv_groups, R = cfg->heads_per_group, K = cfg->topk;
    const int nsplit = msa::decode_splits(cfg, B);
    const int64_t units = (int64_t)B * G;
    auto launch = [&](auto kern, int waves) {
        kern<<<(unsigned)(units * nsplit), waves * 64, 0, st>>>(
            static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k_cache),
            static_cast<const bf16_t *>(v_cache), kv_lens, pooled, nb_max, sel, sel_scores, G, R,
            Nmax, K, nsplit, scale_log2_of(cfg), part_o, part_ml, counters,
            static_cast<bf16_t *>(out), lse);
    };
    if (msa::decode_waves(cfg, B) == 16)
        launch(sparse_decode_kernel<16>, 16);
    else
        launch(sparse_decode_kernel<8>, 8);
    msa_status s = launch_status("sparse decode kernel");
    if (s != MSA_OK || counters) return s;
    combine_kernel<<<(unsigned)(units * R), D, 0, st>>>(part_o, part_ml, G, R, nsplit,
                                                        static_cast<bf16_t *>(out), lse);
    return launch_status("combine kernel");
}

}  // namespace

namespace msa {

// Pooled block scores of every row: the streaming kernel for T*G <= 16, the
// MFMA prefill kernel otherwise; bf16 or OCP E4M3 index data.
msa_status launch_pooled(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                         const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                         const int32_t *q_start, float *pooled, int64_t nb_max, hipStream_t st,
                         int32_t *zero_counters, uint32_t *unpublish, int64_t n_unpublish) {
    const int G = cfg->num_kv_groups;
    const int rows = T * G;
    const bool f8 = cfg->index_dtype == MSA_FP8_E4M3;
    const unsigned char *qi = static_cast<const unsigned char *>(q_idx);
    const unsigned char *ki = static_cast<const unsigned char *>(k_idx);
    if (rows <= msa::kScanMaxRows) {
        const int64_t per_wg = scan_blocks_per_wg(B, nb_max);
        const dim3 grid((unsigned)((nb_max + per_wg - 1) / per_wg), (unsigned)B);
        // Index keys that do not fit the last-level cache are streamed past
        // it (nontemporal loads); a cache that fits stays there between calls.
        const bool stream = (int64_t)B * Nmax * DI * (f8 ? 1 : 2) > kLastLevelCacheBytes;
        auto launch = [&](auto kern) {
            kern<<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G, Nmax, nb_max,
                                       (int)per_wg, zero_counters, unpublish, n_unpublish);
        };
        if (f8)
            stream ? launch(idx_scan_kernel<true, true>) : launch(idx_scan_kernel<true, false>);
        else
            stream ? launch(idx_scan_kernel<false, true>) : launch(idx_scan_kernel<false, false>);
        return launch_status("decode index kernel");
    }
    if (zero_counters) {
        // The MFMA index kernel does not reset the decode attention state.
        const int64_t n = (int64_t)B * G;
        fill_u32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
            reinterpret_cast<uint32_t *>(zero_counters), n, 0u);
        if (unpublish)
            fill_u32_kernel<<<(unsigned)((n_unpublish + 255) / 256), 256, 0, st>>>(
                unpublish, n_unpublish, kUnpublished);
        msa_status s = launch_status("decode state reset kernel");
        if (s != MSA_OK) return s;
    }
    return launch_prefill_pooled(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, pooled, nb_max,
                                 st);
}

// msa_index_topk for T*G <= kScanMaxRows (pooled scores from the streaming
// kernel) or K > kPrefillRegTopk (from the MFMA prefill kernel): pooled scores
// into the workspace, then a wavefront per row ranks them.
msa_status launch_scan_topk(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                            const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                            const int32_t *q_start, int32_t *sel, float *sel_scores,
                            void *workspace, hipStream_t st) {
    const int G = cfg->num_kv_groups, K = cfg->topk;
    const msa::IndexWs w = msa::index_ws(cfg, B, T, Nmax);
    float *pooled = reinterpret_cast<float *>(static_cast<char *>(workspace) + w.pooled_off);
    msa_status s = launch_pooled(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, pooled, w.nb_max, st);
    if (s != MSA_OK) return s;
    const int64_t nrows = (int64_t)B * T * G;
    topk_rows_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(
        pooled, w.nb_max, kv_lens, q_start, B, T, G, Nmax, K, sel, sel_scores);
    return launch_status("top-k kernel");
}

}  // namespace msa

extern "C" {

msa_status msa_sparse_attn_decode(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                                  const void *k_cache, const void *v_cache,
                                  const int32_t *kv_lens, const int32_t *sel, void *out,
                                  float *lse, void *workspace, size_t ws_bytes, void *stream) {
    msa::clear_error();
    msa_status s = msa::check_sparse_args(cfg, B, 1, Nmax, q, k_cache, v_cache, kv_lens, nullptr,
                                          sel, out, lse, workspace, ws_bytes,
                                          MSA_WS_SPARSE_DECODE);
    if (s != MSA_OK || B == 0) return s;
    const msa::DecodeWs w = msa::decode_ws(cfg, B, Nmax, false);
    char *base = static_cast<char *>(workspace);
    return launch_decode_attention(cfg, B, Nmax, q, k_cache, v_cache, kv_lens, nullptr, 0,
                                   const_cast<int32_t *>(sel), nullptr, out, lse,
                                   reinterpret_cast<float *>(base + w.part_o_off),
                                   reinterpret_cast<float *>(base + w.part_ml_off),
                                   reinterpret_cast<hipStream_t>(stream));
}

msa_status msa_decode(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                      const void *q_idx, const void *k_idx, const void *k_cache,
                      const void *v_cache, const int32_t *kv_lens, int32_t *sel,
                      float *sel_scores, void *out, float *lse, void *workspace, size_t ws_bytes,
                      void *stream) {
    msa::clear_error();
    msa_status s = msa::check_decode_args(cfg, B, Nmax, q, q_idx, k_idx, k_cache, v_cache,
                                          kv_lens, sel, sel_scores, out, lse, workspace,
                                          ws_bytes);
    if (s != MSA_OK || B == 0) return s;
    return msa::decode_step(cfg, B, Nmax, q, q_idx, k_idx, k_cache, v_cache, kv_lens, sel,
                            sel_scores, out, lse, static_cast<char *>(workspace),
                            reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace msa {

// The launches of one decode step (msa_decode) on checked arguments, with the
// step's scratch memory (layout decode_ws(cfg, B, Nmax, true)) at `base`.
msa_status decode_step(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                       const void *q_idx, const void *k_idx, const void *k_cache,
                       const void *v_cache, const int32_t *kv_lens, int32_t *sel,
                       float *sel_scores, void *out, float *lse, char *base, hipStream_t st) {
    msa_status s;
    const msa::DecodeWs w = msa::decode_ws(cfg, B, Nmax, true);
    float *pooled = reinterpret_cast<float *>(base + w.pooled_off);
    int32_t *counters = reinterpret_cast<int32_t *>(base + w.counters_off);
    // The split partials, O then (m, l), are one contiguous run of words.
    const int64_t n_part = (int64_t)B * cfg->num_kv_groups * msa::decode_splits(cfg, B) *
                           cfg->heads_per_group * (D + 2);
    s = msa::launch_pooled(cfg, B, 1, Nmax, q_idx, k_idx, kv_lens, nullptr, pooled, w.nb_max, st,
                           counters, reinterpret_cast<uint32_t *>(base + w.part_o_off), n_part);
    if (s != MSA_OK) return s;
    // The attention kernel ranks each (sequence, group) row itself from the
    // pooled scores, attends over the kept blocks, and the last split of each
    // (sequence, group) merges the partials.
    return launch_decode_attention(cfg, B, Nmax, q, k_cache, v_cache, kv_lens, pooled, w.nb_max,
                                   sel, sel_scores, out, lse,
                                   reinterpret_cast<float *>(base + w.part_o_off),
                                   reinterpret_cast<float *>(base + w.part_ml_off), st, counters);
}

}  // namespace msa

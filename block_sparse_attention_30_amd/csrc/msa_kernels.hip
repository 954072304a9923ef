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
//   idx_scan_kernel      decode index scores: streams k_idx once for all
//                        groups through LDS, 16x16x32 bf16 MFMA, causal block
//                        max in registers; writes pooled scores.
//   topk_rows_kernel     one wavefront per row: bitonic sorts of 64-bit keys
//                        (score, inverted block id) across lanes plus
//                        compaction of candidates above a threshold.
//   idx_prefill_kernel   prefill index scores: 32x32x16 bf16 (or 32x32x64
//                        E4M3) MFMA over a 256-row tile with the k_idx block
//                        staged in LDS; block max-pool and a per-row running
//                        top-K in registers in the epilogue.
//   sparse_attn_kernel   (small prefill) one workgroup per (row, group):
//                        gathers the kept 128-token K/V blocks, serves all R
//                        heads of the group with 16x16x32 MFMA (QK^T and PV)
//                        and an online fp32 softmax.
//   pf_*_kernel          (prefill) KV-major sparse attention: per-block entry
//                        lists, one staged block per workgroup serving every
//                        (row, head) that kept it, log-sum-exp merge.
//   sparse_decode_kernel (decode) one 8-wave workgroup per (sequence, group,
//                        split), one 32-token chunk per wave; optionally ranks
//                        the row's blocks itself; waves merge in LDS into a
//                        partial per split; with arrival counters (msa_decode)
//                        the last split of a (sequence, group) merges them all.
//   combine_kernel       (msa_sparse_attn_decode) log-sum-exp merge of the
//                        split partials.
//   fill_i32_kernel      zeroes the prefill list counters (no memset, so the
//                        calls can be captured in graphs).
//   cache_append_kernel  (msa_cache_append) copies new K, V and index-key rows
//                        into the caches, one wavefront per (sequence, row).
//   idx_prefill_kernel<.., QB> and qb_attn_kernel  the query-block-shared
//                        selection variant (msa_index_topk_qblock,
//                        msa_sparse_attn_prefill_qblock): one top-K per
//                        128-row query block; attention query-major with an
//                        online softmax over the block's kept blocks.
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
typedef __attribute__((ext_vector_type(4))) short v4i16;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int S = msa::kBlock;
constexpr int D = msa::kHeadDim;
constexpr int DI = msa::kIndexDim;
constexpr int KMAX = msa::kMaxTopk;
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

typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ i32x8 cat_i32x8(u32x4 lo, u32x4 hi) {
    const i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return r;
}

// OCP E4M3 operands (format code 0 for A and B) with unit block scales (E8M0
// exponent 127 = 1.0): 32 key bytes per lane, lane groups take consecutive
// 32-byte slices of K (A and B use the same slice mapping).
__device__ __forceinline__ f32x4 mfma16_f8(i32x8 a, i32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ f32x16 mfma32_f8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ int clamp_kv(int kv, int Nmax) { return kv < Nmax ? kv : Nmax; }

// floor(a / b) for b > 0 (C division truncates toward zero).
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// Two fp32 values rounded to bf16 (nearest even) and packed, low half first:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// 2^x with the hardware instruction (no denormal rescaling; arguments here
// are <= 0, where that only moves results below 2^-126 to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16_t to_bf16(float v) {
    const __bf16 h = (__bf16)v;
    return __builtin_bit_cast(bf16_t, h);
}

// ---------------------------------------------------------------------------
// Top-k keys. A pooled score and its block id form one unique 64-bit key: the
// fp32 score mapped to an order-preserving uint32 (negative zero taken as
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

// Value of lane (lane ^ J) for a wavefront-uniform J, without LDS traffic.
// J = 1, 2: DPP quad permutation. J = 4, 8: DPP row shifts (row_shl:J gives
// lane i the value of lane i+J, row_shr:J that of lane i-J, within a 16-lane
// row), the upward one where bit J of the lane id is clear. J = 16, 32:
// v_permlane16_swap / v_permlane32_swap of the value with itself; the first
// result holds the partner's value in lanes whose bit J is set, the second in
// lanes whose bit J is clear.
template <int J>
__device__ __forceinline__ uint32_t xor_lane32(uint32_t v, int lane) {
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
    } else if constexpr (J == 4 || J == 8) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x100 + J, 0xF, 0xF, true);
        const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x110 + J, 0xF, 0xF, true);
        return (lane & J) ? dn : up;
    } else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        static_assert(J == 32, "lane distance");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}

// Max / sum of a float over the lanes l, l^16, l^32, l^48 (VALU lane swaps).
__device__ __forceinline__ float max_xor16_32(float v, int lane) {
    v = fmaxf(v, __uint_as_float(xor_lane32<16>(__float_as_uint(v), lane)));
    return fmaxf(v, __uint_as_float(xor_lane32<32>(__float_as_uint(v), lane)));
}

__device__ __forceinline__ float sum_xor16_32(float v, int lane) {
    v += __uint_as_float(xor_lane32<16>(__float_as_uint(v), lane));
    return v + __uint_as_float(xor_lane32<32>(__float_as_uint(v), lane));
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, int lane) {
    const uint32_t lo = xor_lane32<J>((uint32_t)v, lane);
    const uint32_t hi = xor_lane32<J>((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t x, int lane) {
    const uint64_t y = xor_lane64<J>(x, lane);
    const bool keep_max = ((lane & J) == 0) == ((lane & K) == 0);
    return keep_max ? (x > y ? x : y) : (x < y ? x : y);
}

// Bitonic sort of one key per lane across the 64-lane wavefront, descending
// (lane 0 ends with the largest key).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x, int lane) {
    x = bitonic_step<2, 1>(x, lane);
    x = bitonic_step<4, 2>(x, lane);
    x = bitonic_step<4, 1>(x, lane);
    x = bitonic_step<8, 4>(x, lane);
    x = bitonic_step<8, 2>(x, lane);
    x = bitonic_step<8, 1>(x, lane);
    x = bitonic_step<16, 8>(x, lane);
    x = bitonic_step<16, 4>(x, lane);
    x = bitonic_step<16, 2>(x, lane);
    x = bitonic_step<16, 1>(x, lane);
    x = bitonic_step<32, 16>(x, lane);
    x = bitonic_step<32, 8>(x, lane);
    x = bitonic_step<32, 4>(x, lane);
    x = bitonic_step<32, 2>(x, lane);
    x = bitonic_step<32, 1>(x, lane);
    x = bitonic_step<64, 32>(x, lane);
    x = bitonic_step<64, 16>(x, lane);
    x = bitonic_step<64, 8>(x, lane);
    x = bitonic_step<64, 4>(x, lane);
    x = bitonic_step<64, 2>(x, lane);
    x = bitonic_step<64, 1>(x, lane);
    return x;
}

// Top-K of one row by a single wavefront, K <= 32. `cand` holds the row's n
// pooled scores; `buf` is 64 keys of this wave's LDS.
//   Pass 1: every lane takes the best key of its strided share. The K best of
//           those 64 lane maxima are a valid running top-K, and the K-th is a
//           threshold below which no key can enter.
//   Pass 2: keys above the threshold that are not their lane's maximum (those
//           were ranked in pass 1) are appended to the LDS list; when the
//           list is full, or at the end, the list and the current top-K are
//           sorted together and the threshold rises.
// On random scores pass 2 finds only a handful of keys: a row costs two
// 64-key sorts and one read of its scores (two if n > 1024). Returns the K
// best keys in lanes 0..K-1 (descending), 0 elsewhere.
// n_load (>= n) entries of cand may be read: the first batch is loaded
// before n is known to be positive, so its loads can be issued at once.
__device__ __forceinline__ uint64_t wave_topk_row(const float *cand, int n, int n_load, int K,
                                                  int lane, uint64_t *buf) {
    constexpr int kBatch = 16;
    const bool one_batch = n <= 64 * kBatch;  // then pass 2 reuses pass 1's registers
    float v[kBatch];
    auto load = [&](int base) {
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int i = base + c * 64 + lane;
            v[c] = i < n_load ? cand[i] : 0.f;
        }
    };
    uint64_t lmax = 0;
    load(0);
    for (int base = 0; base < n; base += 64 * kBatch) {
        if (base > 0) load(base);
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int i = base + c * 64 + lane;
            const uint64_t k = i < n ? score_key(v[c], i) : 0;
            lmax = k > lmax ? k : lmax;
        }
    }
    const uint64_t srt = wave_sort_desc(lmax, lane);
    uint64_t top = lane < K ? srt : 0;
    uint64_t thr = shfl_u64(srt, K - 1);
    const int cap = 64 - K;
    const uint64_t below = (1ull << lane) - 1ull;
    int cnt = 0;  // wavefront-uniform
    auto merge = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the list writes have landed
        __builtin_amdgcn_wave_barrier();
        uint64_t x = lane < K ? top : ((lane - K) < cnt ? buf[lane - K] : 0);
        x = wave_sort_desc(x, lane);
        top = lane < K ? x : 0;
        thr = shfl_u64(x, K - 1);
        cnt = 0;
        __builtin_amdgcn_wave_barrier();
    };
    if (one_batch) {
        // Usual case: every lane counts its keys above the threshold (other
        // than its maximum, already ranked); a wave prefix sum built from
        // five ballots of the count bits places them in the list at once.
        int my = 0;
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int i = c * 64 + lane;
            const uint64_t kk = i < n ? score_key(v[c], i) : 0;
            my += (kk > thr && kk != lmax) ? 1 : 0;
        }
        int excl = 0, total = 0;
#pragma unroll
        for (int bit = 0; bit < 5; ++bit) {  // my <= 16
            const uint64_t bm = __ballot((my >> bit) & 1);
            excl += __popcll(bm & below) << bit;
            total += __popcll(bm) << bit;
        }
        if (total <= cap) {
            int pos = excl;
#pragma unroll
            for (int c = 0; c < kBatch; ++c) {
                const int i = c * 64 + lane;
                const uint64_t kk = i < n ? score_key(v[c], i) : 0;
                if (kk > thr && kk != lmax) buf[pos++] = kk;
            }
            cnt = total;
            if (cnt) merge();
            return top;
        }
    }
    for (int base = 0; base < n; base += 64 * kBatch) {
        if (!one_batch) load(base);
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int i = base + c * 64 + lane;
            const uint64_t kk = i < n ? score_key(v[c], i) : 0;
            bool q = kk > thr && kk != lmax;
            uint64_t qm = __ballot(q);
            while (qm) {
                if (cnt == cap) {
                    merge();
                    q = q && kk > thr;
                    qm = __ballot(q);
                    continue;
                }
                const int room = cap - cnt;
                const int rank = __popcll(qm & below);
                const bool take = q && rank < room;
                if (take) buf[cnt + rank] = kk;
                const int nq = __popcll(qm);
                cnt += nq < room ? nq : room;
                q = q && !take;
                qm = __ballot(q);
            }
        }
    }
    if (cnt) merge();
    return top;
}

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

template <bool F8>
__global__ __launch_bounds__(256) void idx_scan_kernel(
    const unsigned char *__restrict__ q_idx, const unsigned char *__restrict__ k_idx,
    const int32_t *__restrict__ kv_lens, const int32_t *__restrict__ q_start,
    float *__restrict__ pooled, int T, int G, int Nmax, int64_t nb_max, int blocks_per_wg,
    int32_t *__restrict__ zero_counters) {
    typedef ScanGeom<F8> Geo;
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * Geo::kWaveLds];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Zero the arrival counters the decode attention kernel of the same call
    // uses (one per (sequence, group)); the kernel boundary orders the two.
    if (zero_counters && blockIdx.x == 0)
        for (int i = threadIdx.x; i < G; i += 256) zero_counters[(int64_t)b * G + i] = 0;
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
            v[i] = tok < kv ? ld16(kbytes + (size_t)tok * Geo::kRowBytes + lcol) : zero4;
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
        top = wave_topk_row(pooled + row * nb_max, p / S + 1, p / S + 1, K, lane, s_buf[wave]);
    if (lane < K) {
        sel[row * K + lane] = top ? key_block(top) : -1;
        if (sel_scores) sel_scores[row * K + lane] = top ? key_score(top) : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Prefill index scores. A workgroup owns 256 consecutive (query, group) rows
// of one sequence; wave w owns rows [64w, 64w+64) as two 32-column MFMA tiles
// whose index queries stay in registers (B operand). For each causal KV block
// the 128-token k_idx tile is staged once in LDS (rows padded by 16 bytes so
// that 16 lanes reading 16 bytes each hit distinct banks) and read as the A
// operand by all four waves. D lane l holds column (l & 31) and rows
// 8*(i>>2) + 4*(l>>5) + (i&3), so the block max of a column is an in-lane max
// over the four row tiles plus one exchange with lane l^32. bf16 keys use
// 32x32x16 bf16 MFMAs (8 per row tile and column tile), OCP E4M3 keys
// 32x32x64 f8f6f4 MFMAs with unit scales (2 per row tile and column tile).
constexpr int kPfRows = 256;

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
    int32_t *__restrict__ sel, float *__restrict__ sel_scores, int nslots = 0) {
    constexpr int kRowBytes = DI * (F8 ? 1 : 2);
    constexpr int kRow = kRowBytes + 16;
    constexpr int kPieces = S * kRowBytes / 16 / 256;  // 16-byte loads per thread per block
    constexpr int kKs = F8 ? 2 : 8;                     // MFMA K steps over the index dim
    __shared__ __attribute__((aligned(16))) unsigned char lds[S * kRow];
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
    // The next block's k_idx rows are loaded into registers while the current
    // block is being used from LDS.
    u32x4 pre[kPieces];
    // Loads are unconditional (clamped to the last key, kv >= 1 whenever a
    // block exists) and tokens past kv are zeroed afterwards.
    auto load_block = [&](int blk) {
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int piece = tid + 256 * i;
            const int tk = piece / (kRowBytes / 16), c = piece % (kRowBytes / 16);
            const int tok = blk * S + tk;
            pre[i] = ld16(kseq + (size_t)min(tok, kv - 1) * kRowBytes + c * 16);
            if (tok >= kv) pre[i] = zero4;
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
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
        __builtin_amdgcn_s_barrier();        // ... and every other wave's
        if constexpr (QB)
            if (blk > 0) qb_offer(blk - 1);
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int piece = tid + 256 * i;
            const int tk = piece / (kRowBytes / 16), c = piece % (kRowBytes / 16);
            *reinterpret_cast<u32x4 *>(lds + tk * kRow + c * 16) = pre[i];
        }
        if (blk + 1 < nblk) load_block(blk + 1);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the block's LDS rows are written
        __builtin_amdgcn_s_barrier();
        float cm0 = -INFINITY, cm1 = -INFINITY;
        // Two row tiles at a time: four independent accumulator chains.
#pragma unroll
        for (int rp = 0; rp < 2; ++rp) {
            f32x16 acc[2][2] = {};
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int rt = 2 * rp + h2;
                    const unsigned char *ap = lds + (rt * 32 + j) * kRow + ks * kKb + half * (kKb / 2);
                    if constexpr (F8) {
                        const i32x8 a = cat_i32x8(*reinterpret_cast<const u32x4 *>(ap),
                                                  *reinterpret_cast<const u32x4 *>(ap + 16));
                        acc[h2][0] = mfma32_f8(a, cat_i32x8(qb[0][ks][0], qb[0][ks][F8 ? 1 : 0]), acc[h2][0]);
                        acc[h2][1] = mfma32_f8(a, cat_i32x8(qb[1][ks][0], qb[1][ks][F8 ? 1 : 0]), acc[h2][1]);
                    } else {
                        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(ap));
                        acc[h2][0] = mfma32(a, as_bf16x8(qb[0][ks][0]), acc[h2][0]);
                        acc[h2][1] = mfma32(a, as_bf16x8(qb[1][ks][0]), acc[h2][1]);
                    }
                }
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
    if (nblk > 0) load_block(0);
    for (int blk = 0; blk < n_plain; ++blk) do_block(BoolTag<false>{}, blk);
    for (int blk = n_plain; blk < nblk; ++blk) do_block(BoolTag<true>{}, blk);
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

// ---------------------------------------------------------------------------
// Block-sparse attention (prefill and decode share the chunk step).
//
// A kept 128-token block is cut into four 32-token chunks. For one chunk a
// wave computes, with 16x16x32 bf16 MFMA:
//   S^T = K x q^T : A = 16 tokens of K (16 contiguous bytes per lane straight
//                   from the cache), B = the group's query heads (zero above
//                   R). Lane l holds heads (l & 15), tokens 4*(l>>4)+r.
//   online softmax in the log2 domain, fp32;
//   O  += P x V   : A = P, taken from the lane's own S^T values (two 16-token
//                   tiles give 8 tokens), B = V: the chunk is staged row-major
//                   in LDS and read back with the transposing LDS load
//                   (ds_read_b64_tr_b16), which hands lane i of a 16-lane
//                   group element (i % 4) of the 8-byte piece addressed by
//                   lane 4j + i/4, for j = 0..3 - so lanes that address four
//                   d-values of four tokens receive one d-value of each token.
// Every K/V byte a workgroup reads serves all R heads of the group.
constexpr int kVRow = 288;  // bytes per staged V token row: 256 + 32 pad
constexpr int kVWave = 32 * kVRow;

__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char *p) {
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
    return __builtin_bit_cast(u32x2, r);
}

// A wave's online-softmax state: running max and sum of head (lane & 15) and
// O[head 4*(lane>>4) + r][d = dt*16 + (lane & 15)].
struct WaveAttn {
    float m, l;
    f32x4 o[8];
};

__device__ __forceinline__ void wave_attn_init(WaveAttn &st) {
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// B operand of the S^T MFMA: the R query heads of one row and group.
__device__ __forceinline__ void load_query(bf16x8 (&qf)[4], const bf16_t *q_heads, int R,
                                           int lane) {
    const int col = lane & 15, kg = lane >> 4;
    const bf16_t *qp = q_heads + (size_t)(col < R ? col : 0) * D + kg * 8;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qf[kc] = col < R ? ld_bf16x8(qp + kc * 32) : zero_bf16x8();
}

// The global loads of one 32-token chunk [tok0, tok0 + 32): K in the MFMA A
// layout (token col of each 16-token tile), V as 16-byte row pieces; keys
// past p are clamped (K) or zero (V).
struct ChunkRegs {
    u32x4 kr[2][4], vr[8];
};

__device__ __forceinline__ void load_chunk(ChunkRegs &cr, const bf16_t *kg_base,
                                           const bf16_t *vg_base, int tok0, int p, int lane) {
    const int col = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int tok = tok0 + rt * 16 + col;
        const bf16_t *kp = kg_base + (size_t)(tok <= p ? tok : p) * D + kg * 8;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) cr.kr[rt][kc] = ld16(kp + kc * 32);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int piece = lane + 64 * i;
        const int tok = tok0 + (piece >> 4);
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        cr.vr[i] = tok <= p ? ld16(vg_base + (size_t)tok * D + (piece & 15) * 8) : z4;
    }
}

__device__ __forceinline__ void compute_chunk(WaveAttn &st, const bf16x8 (&qf)[4],
                                              const ChunkRegs &cr, int tok0, int p,
                                              float scale_log2, unsigned char *vrows, int lane);

// One 32-token chunk [tok0, tok0 + 32) of a kept block; keys past p are masked.
__device__ __forceinline__ void attend_chunk(WaveAttn &st, const bf16x8 (&qf)[4],
                                             const bf16_t *kg_base, const bf16_t *vg_base,
                                             int tok0, int p, float scale_log2,
                                             unsigned char *vrows, int lane) {
    ChunkRegs cr;
    load_chunk(cr, kg_base, vg_base, tok0, p, lane);
    compute_chunk(st, qf, cr, tok0, p, scale_log2, vrows, lane);
}

__device__ __forceinline__ void compute_chunk(WaveAttn &st, const bf16x8 (&qf)[4],
                                              const ChunkRegs &cr, int tok0, int p,
                                              float scale_log2, unsigned char *vrows, int lane) {
    const int col = lane & 15, kg = lane >> 4;
    const auto &kr = cr.kr;
    const auto &vr = cr.vr;
    f32x4 sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) acc = mfma16(as_bf16x8(kr[rt][kc]), qf[kc], acc);
        sacc[rt] = acc;
    }
    // V chunk into this wave's LDS rows (tokens past p were loaded as zero).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int piece = lane + 64 * i;
        *reinterpret_cast<u32x4 *>(vrows + (piece >> 4) * kVRow + (piece & 15) * 16) = vr[i];
    }
    // Online softmax (log2 domain). Lane holds head `col`, tokens 4*kg + r
    // (tile 0) and 16 + 4*kg + r (tile 1).
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = tok0 + rt * 16 + 4 * kg + r;
            z[rt][r] = tok <= p ? sacc[rt][r] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, z[rt][r]);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(st.m - m_new);
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
    st.l = st.l * alpha + psum;
    st.m = m_new;
    float a_row[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a_row[r] = __shfl(alpha, 4 * kg + r);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the V rows have landed
    __builtin_amdgcn_wave_barrier();
    // Lane (i, kg) addresses d-values dt*16 + 4*(i&3) .. +3 of tokens
    // 4*kg + (i>>2) and 16 + 4*kg + (i>>2); the transposing read returns
    // d = dt*16 + i of tokens 4*kg + 0..3 and 16 + 4*kg + 0..3, the same token
    // order as the P operand.
    const unsigned char *vlo = vrows + (4 * kg + (col >> 2)) * kVRow + (col & 3) * 8;
    const unsigned char *vhi = vlo + 16 * kVRow;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const u32x2 lo = lds_read_tr16(vlo + dt * 32);
        const u32x2 hi = lds_read_tr16(vhi + dt * 32);
        const u32x4 vb = {lo[0], lo[1], hi[0], hi[1]};
        f32x4 acc = st.o[dt];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= a_row[r];
        st.o[dt] = mfma16(pa, as_bf16x8(vb), acc);
    }
    __builtin_amdgcn_wave_barrier();
}

// Kept blocks of a row, in slot order: ids outside the row's causal range
// (p/S + 1 blocks) are ignored and a repeated id counts once. Called by one
// whole wavefront: lane k checks slot k against the earlier slots, then the
// survivors are compacted by ballot. Returns the count (in every lane).
__device__ __forceinline__ int build_block_list(const int *sel_lds, int K, int p, int *blocks,
                                                int lane, bool unique = false) {
    const int n_valid = p >= 0 ? p / S + 1 : 0;
    bool keep = false;
    int blk = -1;
    if (lane < K) {
        blk = sel_lds[lane];
        keep = blk >= 0 && blk < n_valid;
        // unique: the list comes from this library's own top-k (no repeats).
        if (!unique)
            for (int k2 = 0; k2 < lane && keep; ++k2) keep = sel_lds[k2] != blk;
    }
    const uint64_t m = __ballot(keep);
    if (keep) blocks[__popcll(m & ((1ull << lane) - 1ull))] = blk;
    return __popcll(m);
}

// Merges the NW waves' states by log-sum-exp and writes the R heads' rows of
// out (bf16) and lse (natural log). s_m, s_l: [NW][16] fp32; s_o: [NW][16][128]
// fp32 (may alias the V staging area: the caller has finished with it).
template <int NW>
__device__ __forceinline__ void merge_and_store(const WaveAttn &st, int R, float *s_m, float *s_l,
                                                float *s_o, bf16_t *out_heads, float *lse_heads) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kg = lane >> 4;
    if (lane < 16) {
        s_m[wave * 16 + lane] = st.m;
        s_l[wave * 16 + lane] = st.l;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * kg + r;
        if (h >= R) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w * 16 + h]);
        const float mw = s_m[wave * 16 + h];
        const float sc = mw == -INFINITY ? 0.f : exp2f(mw - M);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) s_o[(wave * 16 + h) * D + dt * 16 + col] = st.o[dt][r] * sc;
    }
    __syncthreads();
    for (int idx = tid; idx < R * D; idx += NW * 64) {
        const int h = idx / D, dd = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w * 16 + h]);
        float Lsum = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            if (s_m[w * 16 + h] != -INFINITY) Lsum += exp2f(s_m[w * 16 + h] - M) * s_l[w * 16 + h];
            acc += s_o[(w * 16 + h) * D + dd];
        }
        out_heads[(size_t)h * D + dd] = to_bf16(Lsum > 0.f ? acc / Lsum : 0.f);
        if (lse_heads && dd == 0) lse_heads[h] = Lsum > 0.f ? M * kLn2 + logf(Lsum) : -INFINITY;
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

__device__ __forceinline__ bool slot_kept(const int32_t *sel_row, int k, int n_valid) {
    const int blk = sel_row[k];
    if (blk < 0 || blk >= n_valid) return false;
    for (int k2 = 0; k2 < k; ++k2)
        if (sel_row[k2] == blk) return false;
    return true;
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t *__restrict__ p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

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

// Row position helper shared by the pass kernels: returns p (or -1 when the
// row is outside the cache or past T).
__device__ __forceinline__ int pf_row_pos(const int32_t *kv_lens, const int32_t *q_start, int b,
                                          int t, int T, int Nmax) {
    if (t >= T) return -1;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    const int p = qs + t;
    return (p >= 0 && p < kv) ? p : -1;
}

// List build of a pass: a counting sort of the kept (row, group, slot)
// entries by block that keeps row order inside every list, so lists and tiles
// come out the same on every run (the backward sums over them):
//   pf_mark_kernel     sets bit tl of the kept block's row bitmap (an atomic
//                      OR, whose result does not depend on the order);
//   pf_rank_kernel     per list: exclusive prefix popcounts of its bitmap
//                      words and its entry count;
//   pf_scan_kernel     list offsets and tiles;
//   pf_scatter_kernel  an entry's rank is its word's prefix plus the popcount
//                      of the lower bits of its word.
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

// Wave per list.
__global__ __launch_bounds__(256) void pf_rank_kernel(const uint32_t *__restrict__ bits,
                                                      int64_t nlists, int W,
                                                      int32_t *__restrict__ wpre,
                                                      int32_t *__restrict__ counts) {
    const int64_t li = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (li >= nlists) return;
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
// their tile counts, and the tile -> list map.
__global__ __launch_bounds__(1024) void pf_scan_kernel(const int32_t *__restrict__ counts,
                                                       int64_t n, int ch,
                                                       int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ tile_first,
                                                       int32_t *__restrict__ tile_map) {
    __shared__ int32_t s_e[1024], s_t[1024];
    const int tid = threadIdx.x;
    const int64_t per = (n + 1023) / 1024;
    const int64_t a = min(n, (int64_t)tid * per), e = min(n, a + per);
    int32_t se = 0, st = 0;
    for (int64_t i = a; i < e; ++i) {
        const int32_t c = counts[i];
        se += c;
        st += (c + ch - 1) / ch;
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
    int32_t oe = s_e[tid] - se, ot = s_t[tid] - st;
    for (int64_t i = a; i < e; ++i) {
        const int32_t c = counts[i], nt = (c + ch - 1) / ch;
        offsets[i] = oe;
        tile_first[i] = ot;
        for (int32_t j = 0; j < nt; ++j) tile_map[ot + j] = (int32_t)i;
        oe += c;
        ot += nt;
    }
    if (tid == 1023) {
        offsets[n] = s_e[1023];
        tile_first[n] = s_t[1023];
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
    list[offsets[li] + r] = (tl << 5) | k;
}

// The list build of one pass (rows t0 .. t0 + rows - 1, groups g0 .. g0 + ng - 1).
void build_pass_lists(const msa::PrefillWs &w, char *base, const int32_t *sel,
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
    const int64_t nwords = w.nlists * W;
    const unsigned slot_blocks = (unsigned)((w.nslots + 255) / 256);
    fill_i32_kernel<<<(unsigned)((nwords + 255) / 256), 256, 0, st>>>(
        reinterpret_cast<int32_t *>(bits), nwords, 0);
    pf_mark_kernel<<<slot_blocks, 256, 0, st>>>(sel, kv_lens, q_start, B, T, G, Nmax, K, t0,
                                                w.rows, g0, ng, w.nb_max, W, bits);
    pf_rank_kernel<<<(unsigned)((w.nlists + 3) / 4), 256, 0, st>>>(bits, w.nlists, W, wpre, counts);
    pf_scan_kernel<<<1, 1024, 0, st>>>(counts, w.nlists, w.entries_per_tile, offsets, tile_first,
                                       tile_map);
    pf_scatter_kernel<<<slot_blocks, 256, 0, st>>>(sel, kv_lens, q_start, bits, wpre, offsets, B,
                                                   T, G, Nmax, K, t0, w.rows, g0, ng, w.nb_max, W,
                                                   list);
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
            const int tl = raw >> 5;
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
                (((int64_t)b * rows + (cent[nq] >> 5)) * ng + gl) * K + (cent[nq] & 31);
            float2 *mlp = has && kg == 0 ? part_ml + slot * R + col % R
                                         : reinterpret_cast<float2 *>(trash + 4096) + col;
            *mlp = make_float2(mrow[nq], lrow[nq]);
            unsigned char *op =
                (has ? reinterpret_cast<unsigned char *>(part_o + (slot * R + col % R) * D)
                     : trash + (col % R) * D * 2) +
                16 * (2 * (kg & 1) + (kg >> 1));
#pragma unroll
            for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4 *>(op + 64 * j) = w4[j];
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
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            if (kt % 2 == 0) __builtin_amdgcn_sched_barrier(0);
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
#pragma unroll
        for (int c = 0; c < S / 32; ++c) {
            const int rlo = c * 32 + 4 * kg + (col >> 2);  // rhi = rlo + 16, same swizzle
            const int lp = (col & 3) >> 1, within = (col & 1) * 8;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                if (dt % 4 == 0) __builtin_amdgcn_sched_barrier(0);
                const int off = qb_swz(rlo, dt * 2 + lp) + within;
                const u32x2 lo = lds_read_tr16(v_lds + off);
                const u32x2 hi = lds_read_tr16(v_lds + off + 16 * 256);
                const u32x4 vbv = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int nq = 0; nq < kPfNq; ++nq) o[nq][dt] = mfma16(as_bf16x8(vbv), pa[nq][c], o[nq][dt]);
            }
        }
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
// d-values of one head over the kept slots.
__global__ __launch_bounds__(256) void pf_merge_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const bf16_t *__restrict__ part_o,
    const float2 *__restrict__ part_ml, int T, int G, int R, int Nmax, int K, int t0, int rows,
    int g0, int ng, bf16_t *__restrict__ out, float *__restrict__ lse) {
    __shared__ int32_t s_sel[KMAX];
    __shared__ int32_t s_kept[KMAX];
    __shared__ int32_t s_n;
    __shared__ float2 s_ml[KMAX * msa::kMaxHeadsPerGroup];
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t unit = blockIdx.x;  // (b, tl, gl), group g0 + gl
    const int g = g0 + (int)(unit % ng);
    const int64_t btl = unit / ng;
    const int b = (int)(btl / rows), tl = (int)(btl % rows);
    const int t = t0 + tl;
    if (t >= T) return;
    const int p = pf_row_pos(kv_lens, q_start, b, t, T, Nmax);
    if (tid < K) s_sel[tid] = p >= 0 ? sel[(((int64_t)b * T + t) * G + g) * K + tid] : -1;
    __syncthreads();
    if (tid < 64) {
        const bool keep = lane < K && p >= 0 && slot_kept(s_sel, lane, p / S + 1);
        const uint64_t m = __ballot(keep);
        if (keep) s_kept[__popcll(m & ((1ull << lane) - 1ull))] = lane;
        if (lane == 0) s_n = __popcll(m);
    }
    __syncthreads();
    const int n = s_n;
    const int64_t slot0 = unit * K;
    for (int i = tid; i < n * R; i += 256) s_ml[i] = part_ml[(slot0 + s_kept[i / R]) * R + i % R];
    __syncthreads();
    const int H = G * R;
    for (int idx = tid; idx < R * (D / 4); idx += 256) {
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

// ---------------------------------------------------------------------------
// Backward of the sparse branch for fixed selections (the Tencent article,
// §五: the two-branch design trains end to end; the selection itself carries
// no gradient). With the forward's lse, P_j = exp2(s_j * tau*log2e -
// lse*log2e) needs no second softmax pass, and with delta = dout . out per
// (row, head), dS_j = P_j (dP_j - delta). Per pass of the forward's list
// build (same lists, tiles and slots):
//   bwd_tile_kernel   one workgroup per tile, each of 8 waves owns 16 keys of
//                     the block with their K and V rows in registers: for each
//                     batch of 64 columns staged in LDS (two buffers), S = q
//                     K^T, dP = dout V^T, dS, then dv^T += dout^T P and dk^T
//                     += q^T dS (the columns as the reduction index); the
//                     batch's dS goes to LDS, where dq^T = K^T dS^T over the
//                     block's 128 keys gives tau * dq per (row, group, slot,
//                     head), bf16; an fp32 [dk; dv] partial per tile;
//   bwd_dkdv_reduce_kernel  per list: dk, dv = sum of its tiles' partials in
//                     tile order (added to the earlier passes' values);
//   bwd_dq_merge_kernel  dq of a (row, group) = fp32 sum of its kept slots'
//                     partials.
// delta comes first from bwd_delta_kernel. No floating-point atomics: every
// sum has one owner and a fixed order.
typedef __attribute__((ext_vector_type(4))) short v4i16;

__device__ __forceinline__ v4i16 pack_bf16x4(float a, float b, float c, float d) {
    const uint32_t lo = pack_bf16x2(a, b), hi = pack_bf16x2(c, d);
    return __builtin_bit_cast(v4i16, u32x2{lo, hi});
}

// delta[r] = sum_d dout[r, d] * out[r, d] for every (row, head) r: 16 lanes per
// r, 16 bytes of each operand per lane.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const bf16_t *__restrict__ out,
                                                        const bf16_t *__restrict__ dout,
                                                        int64_t nrows, float *__restrict__ delta) {
    const int lane = threadIdx.x & 63;
    const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
    const int c = lane & 15;
    float acc = 0.f;
    if (r < nrows) {
        const u32x4 a = ld16(out + r * D + c * 8), d = ld16(dout + r * D + c * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc += __uint_as_float(a[i] << 16) * __uint_as_float(d[i] << 16);
            acc += __uint_as_float(a[i] & 0xFFFF0000u) * __uint_as_float(d[i] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
    if (r < nrows && c == 0) delta[r] = acc;
}

constexpr int kBwdCols = 64;  // columns (entry heads) per bwd_tile_kernel batch
// Columns of one tile: entries_per_tile * R, the same for every R.
constexpr int kBwdTileCols = msa::kPfRounds * msa::kPfWaves * msa::kPfNq * 16;
constexpr int kDsRow = 160;  // bytes per staged dS key row: 64 bf16 columns + 32 pad

constexpr int kBwdWaves = 8;  // bwd_tile_kernel: wave w owns keys 16w .. 16w+15 of the block
constexpr int kBwdKt = 128 / 16 / kBwdWaves;  // 16-key tiles per wave
constexpr int kBwdThreads = kBwdWaves * 64;

__global__ __launch_bounds__(kBwdThreads, 1) void bwd_tile_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache,
    const bf16_t *__restrict__ v_cache, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const float *__restrict__ lse,
    const bf16_t *__restrict__ dout, const float *__restrict__ delta,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ tile_first,
    const int32_t *__restrict__ tile_map, const int32_t *__restrict__ list, int64_t nlists, int T,
    int G, int R, int Nmax, int K, int t0, int rows, int g0, int ng, int64_t nb_max, int ch,
    float scale_log2, float tau, bf16_t *__restrict__ part_dq, float *__restrict__ part_kv,
    unsigned char *__restrict__ trash) {
    // Two buffers of a batch's q and dout rows: batch i+1 is staged into one
    // while batch i is read from the other, one barrier per batch.
    __shared__ __attribute__((aligned(16))) unsigned char q_buf[2][kBwdCols * kVRow];
    __shared__ __attribute__((aligned(16))) unsigned char do_buf[2][kBwdCols * kVRow];
    // Per tile column (entry e, head r at column e*R + r): lse in log2 units,
    // delta, the query position and the dq partial's slot (-1: none).
    __shared__ __attribute__((aligned(16))) float s_lse2[kBwdTileCols], s_dl[kBwdTileCols];
    __shared__ __attribute__((aligned(16))) int s_pc[kBwdTileCols], s_slot[kBwdTileCols];
    // The block's K rows (read transposed for dq) and a batch's dS, one row of
    // 64 bf16 columns per key.
    __shared__ __attribute__((aligned(16))) unsigned char k_s[S * kVRow];
    __shared__ __attribute__((aligned(16))) unsigned char ds_s[S * kDsRow];
    const int w = blockIdx.x;
    if (w >= tile_first[nlists]) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kg = lane >> 4;
    const int li = tile_map[w];
    const int beg = offsets[li] + (w - tile_first[li]) * ch;
    const int nent = min(beg + ch, offsets[li + 1]) - beg;
    const int64_t bgl = li / nb_max;
    const int blk = (int)(li % nb_max);
    const int b = (int)(bgl / ng), gl = (int)(bgl % ng), g = g0 + gl;
    const int64_t bg = (int64_t)b * G + g;
    const int H = G * R;
    const int kv = clamp_kv(kv_lens[b], Nmax);
    const int qs = q_start ? q_start[b] : kv - T;
    // This wave's keys: blk*S + 16*(KT*wave + kt2) + col.
    constexpr int KT = kBwdKt;
    u32x4 kb[KT][4], vb[KT][4];
#pragma unroll
    for (int kt2 = 0; kt2 < KT; ++kt2) {
        const int key = blk * S + 16 * (KT * wave + kt2) + col;
        const bool in = key < kv;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const u32x4 z4 = {0u, 0u, 0u, 0u};
            kb[kt2][kc] = in ? ld16(k_cache + (bg * Nmax + key) * D + kc * 32 + kg * 8) : z4;
            vb[kt2][kc] = in ? ld16(v_cache + (bg * Nmax + key) * D + kc * 32 + kg * 8) : z4;
        }
    }
#pragma unroll
    for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
            *reinterpret_cast<u32x4 *>(k_s + (16 * (KT * wave + kt2) + col) * kVRow + kc * 64 + kg * 16) =
                kb[kt2][kc];
    f32x4 dka[KT][8], dva[KT][8];
#pragma unroll
    for (int kt2 = 0; kt2 < KT; ++kt2)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) dka[kt2][dt] = dva[kt2][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Batches of kBwdCols tile columns: column c of the batch at cb is tile
    // column cb + c, i.e. entry (cb + c) / R, head (cb + c) % R. Thread x of
    // the staging loop owns pieces x, x + kBwdThreads, ... of the batch's
    // 16 x kBwdCols 16-byte pieces (column piece >> 4); the next batch's
    // pieces are loaded into registers while this batch computes.
    constexpr int kSP = kBwdCols * 16 / kBwdThreads;  // pieces per thread
    const int ncol = nent * R;
    for (int tc = tid; tc < kBwdTileCols; tc += kBwdThreads) {
        float l2 = INFINITY, dl = 0.f;
        int pc = -1, slot = -1;
        if (tc < ncol) {
            const int ent = list[beg + tc / R];
            const int64_t hrow = ((int64_t)b * T + t0 + (ent >> 5)) * H + (int64_t)g * R + tc % R;
            l2 = lse[hrow] * kLog2e;
            dl = delta[hrow];
            pc = qs + t0 + (ent >> 5);
            slot = (int)((((int64_t)b * rows + (ent >> 5)) * ng + gl) * K + (ent & 31));
        }
        s_lse2[tc] = l2;
        s_dl[tc] = dl;
        s_pc[tc] = pc;
        s_slot[tc] = slot;
    }
    __syncthreads();
    u32x4 pq[kSP], pd[kSP];
    const int qs_row0 = -qs;  // row in the call = position - q_start
    // A column past the tile's entries loads the last column's data (its
    // position -1 zeroes its P and dS), so the loads are unconditional.
    auto fetch = [&](int cb) {
#pragma unroll
        for (int i = 0; i < kSP; ++i) {
            const int x = tid + kBwdThreads * i, c = x >> 4, piece = x & 15;
            const int tc = min(cb + c, ncol - 1);
            const int64_t hrow = ((int64_t)b * T + qs_row0 + s_pc[tc]) * H + (int64_t)g * R + tc % R;
            pq[i] = ld16(q + hrow * D + piece * 8);
            pd[i] = ld16(dout + hrow * D + piece * 8);
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kSP; ++i) {
            const int x = tid + kBwdThreads * i, c = x >> 4, piece = x & 15;
            *reinterpret_cast<u32x4 *>(q_buf[buf] + c * kVRow + piece * 16) = pq[i];
            *reinterpret_cast<u32x4 *>(do_buf[buf] + c * kVRow + piece * 16) = pd[i];
        }
    };
    if (ncol > 0) {
        fetch(0);
        stage(0);
        if (kBwdCols < ncol) fetch(kBwdCols);
    }
    __syncthreads();
    for (int cb = 0, cur = 0; cb < ncol; cb += kBwdCols, cur ^= 1) {
        // The other buffer was last read in the previous batch, which ended
        // with a barrier.
        if (cb + kBwdCols < ncol) {
            stage(cur ^ 1);
            if (cb + 2 * kBwdCols < ncol) fetch(cb + 2 * kBwdCols);
        }
        const unsigned char *q_s = q_buf[cur];
        const unsigned char *do_s = do_buf[cur];
        const float *b_lse2 = s_lse2 + cb;
        const float *b_dl = s_dl + cb;
        const int *b_pc = s_pc + cb;
#pragma unroll
        for (int cp = 0; cp < kBwdCols / 32; ++cp) {
            // Two 16-column tiles per step: P and dS of both, then one
            // 16x16x32 product per d tile whose k-slots 8*kg .. 8*kg+3 are
            // columns 32*cp + 4*kg + 0..3 and slots 8*kg+4 .. 8*kg+7 columns
            // 32*cp + 16 + 4*kg + 0..3 (the same order in both operands).
            v4i16 pb[2][KT], dsb[2][KT];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int ct = 2 * cp + hf;
                // S = q K^T and dP = dout V^T: lane holds key col of tile kt2
                // and columns 16*ct + 4*kg + r.
                const unsigned char *qrow = q_s + (16 * ct + col) * kVRow + kg * 16;
                const unsigned char *drow = do_s + (16 * ct + col) * kVRow + kg * 16;
#pragma unroll
                for (int kt2 = 0; kt2 < KT; ++kt2) {
                    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, da = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kc = 0; kc < 4; ++kc) {
                        sa = mfma16(as_bf16x8(*reinterpret_cast<const u32x4 *>(qrow + kc * 64)),
                                    as_bf16x8(kb[kt2][kc]), sa);
                        da = mfma16(as_bf16x8(*reinterpret_cast<const u32x4 *>(drow + kc * 64)),
                                    as_bf16x8(vb[kt2][kc]), da);
                    }
                    // Branch-free: exp of every element (a padding column has
                    // lse = +inf, so 0), then the causal select.
                    const int key = blk * S + 16 * (KT * wave + kt2) + col;
                    const int c0 = 16 * ct + 4 * kg;
                    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(b_lse2 + c0);
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(b_dl + c0);
                    const u32x4 p4 = *reinterpret_cast<const u32x4 *>(b_pc + c0);
                    float pv[4], dsv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float e = fast_exp2(fmaf(sa[r], scale_log2, -l4[r]));
                        const float p = key > (int)p4[r] ? 0.f : e;
                        pv[r] = p;
                        dsv[r] = p * (da[r] - d4[r]);
                    }
                    pb[hf][kt2] = pack_bf16x4(pv[0], pv[1], pv[2], pv[3]);
                    dsb[hf][kt2] = pack_bf16x4(dsv[0], dsv[1], dsv[2], dsv[3]);
                    *reinterpret_cast<v4i16 *>(ds_s + (16 * (KT * wave + kt2) + col) * kDsRow +
                                               (16 * ct + 4 * kg) * 2) = dsb[hf][kt2];
                }
            }
            // dv^T += dout^T P and dk^T += q^T dS over these 32 columns:
            // dout^T / q^T read transposed from LDS (column rows 4*kg + i of
            // each half).
            const unsigned char *dt_lo = do_s + (32 * cp + 4 * kg + (col >> 2)) * kVRow + (col & 3) * 8;
            const unsigned char *qt_lo = q_s + (32 * cp + 4 * kg + (col >> 2)) * kVRow + (col & 3) * 8;
            bf16x8 pb8[KT], ds8[KT];
#pragma unroll
            for (int kt2 = 0; kt2 < KT; ++kt2) {
                pb8[kt2] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(pb[0][kt2], pb[1][kt2], 0, 1, 2, 3, 4, 5, 6, 7));
                ds8[kt2] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(dsb[0][kt2], dsb[1][kt2], 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const u32x2 dlo = lds_read_tr16(dt_lo + dt * 32);
                const u32x2 dhi = lds_read_tr16(dt_lo + 16 * kVRow + dt * 32);
                const u32x2 qlo = lds_read_tr16(qt_lo + dt * 32);
                const u32x2 qhi = lds_read_tr16(qt_lo + 16 * kVRow + dt * 32);
                const u32x4 d4 = {dlo[0], dlo[1], dhi[0], dhi[1]};
                const u32x4 q4 = {qlo[0], qlo[1], qhi[0], qhi[1]};
#pragma unroll
                for (int kt2 = 0; kt2 < KT; ++kt2) {
                    dva[kt2][dt] = mfma16(as_bf16x8(d4), pb8[kt2], dva[kt2][dt]);
                    dka[kt2][dt] = mfma16(as_bf16x8(q4), ds8[kt2], dka[kt2][dt]);
                }
            }
        }
        __syncthreads();  // the batch's dS is in LDS
        // dq^T = K^T dS^T for the batch, tau applied: wave w owns column
        // tiles 2*(w&1) + j and d tiles 2*(w>>1) + i; K^T and dS^T are read
        // transposed from LDS, keys 4*kg + 0..3 and 16 + 4*kg + 0..3 of each
        // 32-key chunk in both operands.
        {
            f32x4 dqa[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) dqa[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < S / 32; ++cc) {
                const int krow = cc * 32 + 4 * kg + (col >> 2);
                bf16x8 bq[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const unsigned char *p = ds_s + krow * kDsRow + (2 * (wave & 1) + j) * 32 + (col & 3) * 8;
                    const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 16 * kDsRow);
                    bq[j] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const unsigned char *p = k_s + krow * kVRow + (2 * (wave >> 1) + i) * 32 + (col & 3) * 8;
                    const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 16 * kVRow);
                    const bf16x8 ka = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
                    for (int j = 0; j < 2; ++j) dqa[i][j] = mfma16(ka, bq[j], dqa[i][j]);
                }
            }
            // Lane holds column 16*ct + col, d = 16*dt + 4*kg + r.
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tc = cb + 16 * (2 * (wave & 1) + j) + col;
                const int slot = s_slot[tc];
                // A column without an entry stores into the trash area (no
                // branch, so waits count the same stores on every path).
                bf16_t *op = (slot >= 0 ? part_dq + ((int64_t)slot * R + tc % R) * D
                                        : reinterpret_cast<bf16_t *>(trash) + (tc % R) * D) +
                             4 * kg;
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    *reinterpret_cast<u32x2 *>(op + (2 * (wave >> 1) + i) * 16) =
                        u32x2{pack_bf16x2(tau * dqa[i][j][0], tau * dqa[i][j][1]),
                              pack_bf16x2(tau * dqa[i][j][2], tau * dqa[i][j][3])};
            }
        }
        __syncthreads();  // this batch's buffers are read, the next one is staged
    }
    // The tile's partial: [K rows 0..127][d] then [V rows][d], fp32 (tau not
    // yet applied to dK). Lane holds d = dt*16 + 4*kg + r of key col.
    float *pk = part_kv + (int64_t)w * 2 * S * D;
#pragma unroll
    for (int kt2 = 0; kt2 < KT; ++kt2) {
        const int kr = 16 * (KT * wave + kt2) + col;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            *reinterpret_cast<f32x4 *>(pk + (int64_t)kr * D + dt * 16 + 4 * kg) = dka[kt2][dt];
            *reinterpret_cast<f32x4 *>(pk + (int64_t)(S + kr) * D + dt * 16 + 4 * kg) = dva[kt2][dt];
        }
    }
}

// dk, dv of one list's block: the sum of its tiles' partials in tile order
// (tau applied to dk), added to the earlier passes' values when accumulate;
// a list without entries contributes zero.
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(
    const int32_t *__restrict__ tile_first, const float *__restrict__ part_kv, int G, int Nmax,
    int g0, int ng, int64_t nb_max, float tau, int accumulate, float *__restrict__ dk,
    float *__restrict__ dv) {
    const int64_t li = blockIdx.x;
    const int64_t bgl = li / nb_max;
    const int blk = (int)(li % nb_max);
    const int b = (int)(bgl / ng), g = g0 + (int)(bgl % ng);
    const int64_t bg = (int64_t)b * G + g;
    const int t_lo = tile_first[li], t_hi = tile_first[li + 1];
    if (t_lo == t_hi && accumulate) return;
    // Thread x owns four consecutive floats of one row of K or V, 2*S*D/4
    // groups in all.
    for (int x = threadIdx.x; x < 2 * S * D / 4; x += 256) {
        const int row = x / (D / 4), d0 = (x % (D / 4)) * 4;  // row < S: K, else V
        const int kr = row < S ? row : row - S;
        const int key = blk * S + kr;
        if (key >= Nmax) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int t = t_lo; t < t_hi; ++t)
            acc += *reinterpret_cast<const f32x4 *>(part_kv + ((int64_t)t * 2 * S + row) * D + d0);
        float *dst = (row < S ? dk : dv) + (bg * Nmax + key) * D + d0;
        if (row < S) acc *= tau;
        if (accumulate) acc += *reinterpret_cast<const f32x4 *>(dst);
        *reinterpret_cast<f32x4 *>(dst) = acc;
    }
}

// dq of one (sequence, row of the pass, group): the kept slots' partials
// summed in slot order; zero for a row outside the cache.
__global__ __launch_bounds__(256) void bwd_dq_merge_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const bf16_t *__restrict__ part_dq, int T, int G, int R,
    int Nmax, int K, int t0, int rows, int g0, int ng, float *__restrict__ dq) {
    __shared__ int32_t s_sel[KMAX];
    __shared__ int32_t s_kept[KMAX];
    __shared__ int32_t s_n;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t unit = blockIdx.x;
    const int g = g0 + (int)(unit % ng);
    const int64_t btl = unit / ng;
    const int b = (int)(btl / rows), tl = (int)(btl % rows);
    const int t = t0 + tl;
    if (t >= T) return;
    const int p = pf_row_pos(kv_lens, q_start, b, t, T, Nmax);
    if (tid < K) s_sel[tid] = p >= 0 ? sel[(((int64_t)b * T + t) * G + g) * K + tid] : -1;
    __syncthreads();
    if (tid < 64) {
        const bool keep = lane < K && p >= 0 && slot_kept(s_sel, lane, p / S + 1);
        const uint64_t m = __ballot(keep);
        if (keep) s_kept[__popcll(m & ((1ull << lane) - 1ull))] = lane;
        if (lane == 0) s_n = __popcll(m);
    }
    __syncthreads();
    const int n = s_n;
    const int H = G * R;
    for (int idx = tid; idx < R * (D / 4); idx += 256) {
        const int r = idx / (D / 4), d0 = (idx % (D / 4)) * 4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < n; ++i) {
            const u32x2 pv =
                *reinterpret_cast<const u32x2 *>(part_dq + ((unit * K + s_kept[i]) * R + r) * D + d0);
            acc[0] += __uint_as_float(pv[0] << 16);
            acc[1] += __uint_as_float(pv[0] & 0xFFFF0000u);
            acc[2] += __uint_as_float(pv[1] << 16);
            acc[3] += __uint_as_float(pv[1] & 0xFFFF0000u);
        }
        *reinterpret_cast<f32x4 *>(dq + (((int64_t)b * T + t) * H + (int64_t)g * R + r) * D + d0) = acc;
    }
}

// Decode: the new token of sequence b sits at position kv - 1. Group g's
// kept blocks give 4*nblk 32-token chunks; workgroup (b, g, split) has eight
// waves and takes chunks [8*split, 8*split + 8), one per wave, so every load
// of the split is in flight at once. With `pooled` non-null each workgroup
// first ranks the row itself (wave 0, from the pooled block scores; split 0
// also writes sel / sel_scores), otherwise it reads sel. The waves merge in
// LDS into one unnormalised partial (O, m, l) per split, which
// combine_kernel merges by log-sum-exp.
constexpr int kDecWaves = 8;
constexpr int kDecChunks = kDecWaves;  // chunks per split

struct DecodeLds {
    unsigned char vrows[kDecWaves * kVWave];  // V chunks; then [8][16][128] fp32 outputs
    uint64_t keys[64];                        // top-k list
    int sel[KMAX];
    int blocks[KMAX];
    int nblk;
    float m[kDecWaves * 16], l[kDecWaves * 16];
};

__global__ __launch_bounds__(512) void sparse_decode_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache,
    const bf16_t *__restrict__ v_cache, const int32_t *__restrict__ kv_lens,
    const float *__restrict__ pooled, int64_t nb_max, int32_t *__restrict__ sel,
    float *__restrict__ sel_scores, int G, int R, int Nmax, int K, int nsplit, float scale_log2,
    float *__restrict__ part_o, float *__restrict__ part_ml, int32_t *__restrict__ counters,
    bf16_t *__restrict__ out, float *__restrict__ lse) {
    __shared__ DecodeLds L;
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
        if (wave == 0) {
            // n_load = nb_max: the row's pooled scores are loaded while kv_lens
            // is still in flight.
            const uint64_t top = wave_topk_row(pooled + unit * nb_max, p >= 0 ? p / S + 1 : 0,
                                               (int)nb_max, K, lane, L.keys);
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
    const int c = split * kDecChunks + wave;  // this wave's chunk
    WaveAttn st;
    wave_attn_init(st);
    if (c < L.nblk * 4) {
        attend_chunk(st, qf, k_cache + ((size_t)b * G + g) * Nmax * D,
                     v_cache + ((size_t)b * G + g) * Nmax * D, L.blocks[c >> 2] * S + (c & 3) * 32,
                     p, scale_log2, L.vrows + wave * kVWave, lane);
    }
    // Merge the eight waves into this split's partial.
    float *s_o = reinterpret_cast<float *>(L.vrows);
    const int col = lane & 15, kg = lane >> 4;
    if (lane < 16) {
        L.m[wave * 16 + lane] = st.m;
        L.l[wave * 16 + lane] = st.l;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * kg + r;
        if (h >= R) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, L.m[w * 16 + h]);
        const float mw = L.m[wave * 16 + h];
        const float sc = mw == -INFINITY ? 0.f : exp2f(mw - M);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) s_o[(wave * 16 + h) * D + dt * 16 + col] = st.o[dt][r] * sc;
    }
    __syncthreads();
    for (int idx = tid; idx < R * D; idx += kDecWaves * 64) {
        const int h = idx / D, dd = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, L.m[w * 16 + h]);
        float Lsum = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
            if (L.m[w * 16 + h] != -INFINITY) Lsum += exp2f(L.m[w * 16 + h] - M) * L.l[w * 16 + h];
            acc += s_o[(w * 16 + h) * D + dd];
        }
        const int64_t pu = (unit * nsplit + split) * R + h;
        if (counters) {
            // Device-scope stores: written through to memory, where the
            // merging workgroup (possibly on another XCD) reads them.
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
    // all partials. Every thread's partial stores have completed (vmcnt(0))
    // before the workgroup's arrival is counted; the merging workgroup reads
    // the partials with device-scope loads, after its own arrival.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0)
        L.nblk = __hip_atomic_fetch_add(&counters[unit], 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
    __syncthreads();
    if (!L.nblk) return;
    // One round of loads per batch of eight splits, merged online.
    for (int idx = tid; idx < R * D; idx += kDecWaves * 64) {
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

// Blocks per decode-scan workgroup: about 4096 workgroups over the batch
// (measured best on the 16 x 131072 decode, where it is one block per wave),
// at least 4 (one per wave), a multiple of 4.
int64_t scan_blocks_per_wg(int32_t B, int64_t nb_max) {
    int64_t per = ((int64_t)B * nb_max + 4095) / 4096;
    return per < 4 ? 4 : (per + 3) / 4 * 4;
}

// Pooled block scores of every row: the streaming kernel for T*G <= 16, the
// MFMA prefill kernel otherwise; bf16 or OCP E4M3 index data.
msa_status launch_pooled(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                         const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                         const int32_t *q_start, float *pooled, int64_t nb_max, hipStream_t st,
                         int32_t *zero_counters = nullptr) {
    const int G = cfg->num_kv_groups;
    const int rows = T * G;
    const bool f8 = cfg->index_dtype == MSA_FP8_E4M3;
    const unsigned char *qi = static_cast<const unsigned char *>(q_idx);
    const unsigned char *ki = static_cast<const unsigned char *>(k_idx);
    if (rows <= msa::kScanMaxRows) {
        const int64_t per_wg = scan_blocks_per_wg(B, nb_max);
        const dim3 grid((unsigned)((nb_max + per_wg - 1) / per_wg), (unsigned)B);
        if (f8)
            idx_scan_kernel<true><<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G,
                                                        Nmax, nb_max, (int)per_wg, zero_counters);
        else
            idx_scan_kernel<false><<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G,
                                                         Nmax, nb_max, (int)per_wg, zero_counters);
        return launch_status("decode index kernel");
    }
    const dim3 grid((unsigned)((rows + kPfRows - 1) / kPfRows), (unsigned)B);
    if (f8)
        idx_prefill_kernel<true, 0><<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G,
                                                          Nmax, nb_max, 0, nullptr, nullptr);
    else
        idx_prefill_kernel<false, 0><<<grid, 256, 0, st>>>(qi, ki, kv_lens, q_start, pooled, T, G,
                                                           Nmax, nb_max, 0, nullptr, nullptr);
    return launch_status("prefill index kernel");
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
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int G = cfg->num_kv_groups, K = cfg->topk;
    if (T * G > msa::kScanMaxRows) {
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
    const msa::IndexWs w = msa::index_ws(cfg, B, T, Nmax);
    float *pooled = reinterpret_cast<float *>(static_cast<char *>(workspace) + w.pooled_off);
    s = launch_pooled(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, pooled, w.nb_max, st);
    if (s != MSA_OK) return s;
    const int64_t nrows = (int64_t)B * T * G;
    topk_rows_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(
        pooled, w.nb_max, kv_lens, q_start, B, T, G, Nmax, K, sel, sel_scores);
    return launch_status("top-k kernel");
}

msa_status msa_index_pool(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                          const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                          const int32_t *q_start, float *pooled, void *stream) {
    msa::clear_error();
    msa_status s =
        msa::check_pool_args(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, pooled);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    return launch_pooled(cfg, B, T, Nmax, q_idx, k_idx, kv_lens, q_start, pooled,
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
    int32_t *counts = reinterpret_cast<int32_t *>(base + w.counts_off);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + w.offsets_off);
    int32_t *tile_first = reinterpret_cast<int32_t *>(base + w.tile_first_off);
    int32_t *tile_map = reinterpret_cast<int32_t *>(base + w.tile_map_off);
    int32_t *list = reinterpret_cast<int32_t *>(base + w.list_off);
    bf16_t *part_o = reinterpret_cast<bf16_t *>(base + w.part_o_off);
    float2 *part_ml = reinterpret_cast<float2 *>(base + w.part_ml_off);
    for (int32_t g0 = 0; g0 < G; g0 += w.groups)
      for (int32_t t0 = 0; t0 < T; t0 += w.rows) {
        const int ng = w.groups;
        build_pass_lists(w, base, sel, kv_lens, q_start, B, T, G, Nmax, K, t0, g0, st);
        pf_attn_kernel<<<(unsigned)w.max_tiles, 256, 0, st>>>(
            qp, kp, vp, kv_lens, q_start, offsets, tile_first, tile_map, list, w.nlists, T, G, R,
            Nmax, K, t0, w.rows, g0, ng, w.nb_max, w.entries_per_tile, sl2, part_o, part_ml,
            reinterpret_cast<unsigned char *>(base + w.trash_off));
        pf_merge_kernel<<<(unsigned)((int64_t)B * w.rows * ng), 256, 0, st>>>(
            sel, kv_lens, q_start, part_o, part_ml, T, G, R, Nmax, K, t0, w.rows, g0, ng, op, lse);
        s = launch_status("sparse prefill kernels");
        if (s != MSA_OK) return s;
    }
    return MSA_OK;
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
    const int nsplit = msa::decode_splits(cfg);
    const int64_t units = (int64_t)B * G;
    sparse_decode_kernel<<<(unsigned)(units * nsplit), kDecWaves * 64, 0, st>>>(
        static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(k_cache),
        static_cast<const bf16_t *>(v_cache), kv_lens, pooled, nb_max, sel, sel_scores, G, R, Nmax,
        K, nsplit, scale_log2_of(cfg), part_o, part_ml, counters, static_cast<bf16_t *>(out),
        lse);
    msa_status s = launch_status("sparse decode kernel");
    if (s != MSA_OK || counters) return s;
    combine_kernel<<<(unsigned)(units * R), D, 0, st>>>(part_o, part_ml, G, R, nsplit,
                                                        static_cast<bf16_t *>(out), lse);
    return launch_status("combine kernel");
}

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

msa_status msa_sparse_attn_backward(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                    const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *kv_lens, const int32_t *q_start,
                                    const int32_t *sel, const void *out, const float *lse,
                                    const void *dout, float *dq, float *dk, float *dv,
                                    void *workspace, size_t ws_bytes, void *stream) {
    msa::clear_error();
    msa_status s = msa::check_backward_args(cfg, B, T, Nmax, q, k_cache, v_cache, kv_lens,
                                            q_start, sel, out, lse, dout, dq, dk, dv, workspace,
                                            ws_bytes);
    if (s != MSA_OK || B == 0 || T == 0) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int G = cfg->num_kv_groups, R = cfg->heads_per_group, K = cfg->topk;
    const float sl2 = scale_log2_of(cfg);
    const float tau = sl2 / kLog2e;
    const bf16_t *qp = static_cast<const bf16_t *>(q);
    const bf16_t *kp = static_cast<const bf16_t *>(k_cache);
    const bf16_t *vp = static_cast<const bf16_t *>(v_cache);
    const bf16_t *dop = static_cast<const bf16_t *>(dout);
    const msa::PrefillWs w = msa::prefill_ws(cfg, B, T, Nmax, true);
    char *base = static_cast<char *>(workspace);
    int32_t *counts = reinterpret_cast<int32_t *>(base + w.counts_off);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + w.offsets_off);
    int32_t *tile_first = reinterpret_cast<int32_t *>(base + w.tile_first_off);
    int32_t *tile_map = reinterpret_cast<int32_t *>(base + w.tile_map_off);
    int32_t *list = reinterpret_cast<int32_t *>(base + w.list_off);
    bf16_t *part_dq = reinterpret_cast<bf16_t *>(base + w.part_o_off);
    float *part_kv = reinterpret_cast<float *>(base + w.part_ml_off);
    float *delta = reinterpret_cast<float *>(base + w.delta_off);
    const int64_t nrows = (int64_t)B * T * G * R;
    bwd_delta_kernel<<<(unsigned)((nrows * 16 + 255) / 256), 256, 0, st>>>(
        static_cast<const bf16_t *>(out), dop, nrows, delta);
    for (int32_t g0 = 0; g0 < G; g0 += w.groups)
      for (int32_t t0 = 0; t0 < T; t0 += w.rows) {
        const int ng = w.groups;
        build_pass_lists(w, base, sel, kv_lens, q_start, B, T, G, Nmax, K, t0, g0, st);
        bwd_tile_kernel<<<(unsigned)w.max_tiles, kBwdThreads, 0, st>>>(
            qp, kp, vp, kv_lens, q_start, lse, dop, delta, offsets, tile_first, tile_map, list,
            w.nlists, T, G, R, Nmax, K, t0, w.rows, g0, ng, w.nb_max, w.entries_per_tile, sl2,
            tau, part_dq, part_kv, reinterpret_cast<unsigned char *>(base + w.trash_off));
        bwd_dkdv_reduce_kernel<<<(unsigned)w.nlists, 256, 0, st>>>(
            tile_first, part_kv, G, Nmax, g0, ng, w.nb_max, tau, t0 > 0 ? 1 : 0, dk, dv);
        bwd_dq_merge_kernel<<<(unsigned)((int64_t)B * w.rows * ng), 256, 0, st>>>(
            sel, kv_lens, q_start, part_dq, T, G, R, Nmax, K, t0, w.rows, g0, ng, dq);
        s = launch_status("sparse backward kernels");
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
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const msa::DecodeWs w = msa::decode_ws(cfg, B, Nmax, true);
    char *base = static_cast<char *>(workspace);
    float *pooled = reinterpret_cast<float *>(base + w.pooled_off);
    int32_t *counters = reinterpret_cast<int32_t *>(base + w.counters_off);
    s = launch_pooled(cfg, B, 1, Nmax, q_idx, k_idx, kv_lens, nullptr, pooled, w.nb_max, st,
                      counters);
    if (s != MSA_OK) return s;
    // The attention kernel ranks each (sequence, group) row itself from the
    // pooled scores, attends over the kept blocks, and the last split of each
    // (sequence, group) merges the partials.
    return launch_decode_attention(cfg, B, Nmax, q, k_cache, v_cache, kv_lens, pooled, w.nb_max,
                                   sel, sel_scores, out, lse,
                                   reinterpret_cast<float *>(base + w.part_o_off),
                                   reinterpret_cast<float *>(base + w.part_ml_off), st, counters);
}

}  // extern "C"

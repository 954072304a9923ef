// Device helpers shared by the libmsa kernel sources (gfx950, MI355X): vector
// types, MFMA wrappers, bf16 packing, the wave-level top-k sort, the
// attention chunk step shared by the query-major prefill and the decode
// kernels, and the host launchers one kernel source calls in another.
// Internal to the library; not part of the ABI.
#ifndef MSA_DEVICE_H
#define MSA_DEVICE_H

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "msa_internal.h"

namespace msa {
// Pooled block scores of every row: the streaming decode kernel for
// T*G <= kScanMaxRows, the MFMA prefill kernel otherwise (msa_decode.hip).
msa_status launch_pooled(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                         const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                         const int32_t *q_start, float *pooled, int64_t nb_max, hipStream_t st,
                         int32_t *zero_counters = nullptr, uint32_t *unpublish = nullptr,
                         int64_t n_unpublish = 0);
// The MFMA path of launch_pooled (msa_prefill.hip).
msa_status launch_prefill_pooled(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                                 const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                                 const int32_t *q_start, float *pooled, int64_t nb_max,
                                 hipStream_t st);
// msa_index_topk for T*G <= kScanMaxRows (msa_decode.hip).
msa_status launch_scan_topk(const msa_config *cfg, int32_t B, int32_t T, int32_t Nmax,
                            const void *q_idx, const void *k_idx, const int32_t *kv_lens,
                            const int32_t *q_start, int32_t *sel, float *sel_scores,
                            void *workspace, hipStream_t st);
// The launches of one decode step (msa_decode.hip) on checked arguments, its
// scratch memory (layout decode_ws(cfg, B, Nmax, true)) at `base`: shared by
// msa_decode (caller workspace) and msa_decode_no_alloc (fixed scratch).
msa_status decode_step(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                       const void *q_idx, const void *k_idx, const void *k_cache,
                       const void *v_cache, const int32_t *kv_lens, int32_t *sel,
                       float *sel_scores, void *out, float *lse, char *base, hipStream_t st);
// The KV-major list build of one pass (msa_prefill.hip), shared by the
// sparse prefill and its backward.
void build_pass_lists(const PrefillWs &w, char *base, const int32_t *sel, const int32_t *kv_lens,
                      const int32_t *q_start, int B, int T, int G, int Nmax, int K, int t0,
                      int g0, hipStream_t st);
}  // namespace msa

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
// Streaming 16-byte load for data read once (nontemporal hint): it leaves the
// caches to data that is reused, and a kernel that only streams moves
// measurably more bytes per second with it than with plain loads.
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

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
__device__ __forceinline__ uint32_t score_bits(float s) {
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t score_key(float s, int blk) {
    return ((uint64_t)score_bits(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)blk);
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

// The 64 largest of two descending-sorted lane registers, descending: the
// elementwise max of a and b reversed is a bitonic sequence holding them, and
// the last stage's steps sort it.
__device__ __forceinline__ uint64_t merge_sorted_desc(uint64_t a, uint64_t b, int lane) {
    const uint64_t br = shfl_u64(b, 63 - lane);
    uint64_t x = a > br ? a : br;
    x = bitonic_step<64, 32>(x, lane);
    x = bitonic_step<64, 16>(x, lane);
    x = bitonic_step<64, 8>(x, lane);
    x = bitonic_step<64, 4>(x, lane);
    x = bitonic_step<64, 2>(x, lane);
    return bitonic_step<64, 1>(x, lane);
}

// Top-K of one row by a single wavefront, K <= 64. `cand` holds the row's n
// pooled scores; `buf` is 64 keys of this wave's LDS.
//   Pass 1: every lane takes the best key of its strided share. The K best of
//           those 64 lane maxima are a valid running top-K, and the K-th is a
//           threshold below which no key can enter.
//   Pass 2: keys above the threshold that are not their lane's maximum (those
//           were ranked in pass 1) are appended to the LDS list; when the
//           list is full, or at the end, the list and the current top-K are
//           ranked together and the threshold rises: for K <= 32 the top-K
//           and a list of up to 64 - K keys are sorted as one register; for
//           K > 32 the list (up to 64 keys) is sorted on its own and merged
//           with the top-K register (merge_sorted_desc).
// On random scores pass 2 finds only a handful of keys: a row costs two
// 64-key sorts and one read of its scores (two if n > 1024). Returns the K
// best keys in lanes 0..K-1 (descending), 0 elsewhere.
// n_load (>= n) entries of cand may be read: the first batch is loaded
// before n is known to be positive, so its loads can be issued at once.
// cand[i] is the score of block blk0 + i (keys carry the absolute block id).
__device__ __forceinline__ uint64_t wave_topk_row(const float *cand, int n, int n_load, int K,
                                                  int lane, uint64_t *buf, int blk0 = 0) {
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
            const uint64_t k = i < n ? score_key(v[c], blk0 + i) : 0;
            lmax = k > lmax ? k : lmax;
        }
    }
    const uint64_t srt = wave_sort_desc(lmax, lane);
    uint64_t top = lane < K ? srt : 0;
    uint64_t thr = shfl_u64(srt, K - 1);
    const bool big = K > 32;  // wavefront-uniform
    const int cap = big ? 64 : 64 - K;
    const uint64_t below = (1ull << lane) - 1ull;
    int cnt = 0;  // wavefront-uniform
    auto merge = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the list writes have landed
        __builtin_amdgcn_wave_barrier();
        uint64_t x;
        if (big) {
            const uint64_t y = wave_sort_desc(lane < cnt ? buf[lane] : 0, lane);
            x = merge_sorted_desc(top, y, lane);
        } else {
            x = lane < K ? top : ((lane - K) < cnt ? buf[lane - K] : 0);
            x = wave_sort_desc(x, lane);
        }
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
            const uint64_t kk = i < n ? score_key(v[c], blk0 + i) : 0;
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
                const uint64_t kk = i < n ? score_key(v[c], blk0 + i) : 0;
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
            const uint64_t kk = i < n ? score_key(v[c], blk0 + i) : 0;
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

template <int K, int J>
__device__ __forceinline__ uint32_t bitonic_step_u32(uint32_t x, int lane) {
    const uint32_t y = xor_lane32<J>(x, lane);
    const bool keep_max = ((lane & J) == 0) == ((lane & K) == 0);
    return keep_max ? (x > y ? x : y) : (x < y ? x : y);
}

// Bitonic sort of one 32-bit value per lane, descending.
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t x, int lane) {
    x = bitonic_step_u32<2, 1>(x, lane);
    x = bitonic_step_u32<4, 2>(x, lane);
    x = bitonic_step_u32<4, 1>(x, lane);
    x = bitonic_step_u32<8, 4>(x, lane);
    x = bitonic_step_u32<8, 2>(x, lane);
    x = bitonic_step_u32<8, 1>(x, lane);
    x = bitonic_step_u32<16, 8>(x, lane);
    x = bitonic_step_u32<16, 4>(x, lane);
    x = bitonic_step_u32<16, 2>(x, lane);
    x = bitonic_step_u32<16, 1>(x, lane);
    x = bitonic_step_u32<32, 16>(x, lane);
    x = bitonic_step_u32<32, 8>(x, lane);
    x = bitonic_step_u32<32, 4>(x, lane);
    x = bitonic_step_u32<32, 2>(x, lane);
    x = bitonic_step_u32<32, 1>(x, lane);
    x = bitonic_step_u32<64, 32>(x, lane);
    x = bitonic_step_u32<64, 16>(x, lane);
    x = bitonic_step_u32<64, 8>(x, lane);
    x = bitonic_step_u32<64, 4>(x, lane);
    x = bitonic_step_u32<64, 2>(x, lane);
    return bitonic_step_u32<64, 1>(x, lane);
}

// Top-K (K <= 64) of one row of n pooled scores by one wavefront, the same
// result as wave_topk_row with a shorter dependency chain for n <= 1024: the
// first pass ranks only the score halves of the 64 lane maxima (a 32-bit
// sort); the K-th of them is a score no top-K key lies below, since K lanes
// hold a key at least that large. Every valid key whose score reaches it is a
// candidate; when there are at most 64, they are compacted through `buf` (64
// keys of this wave's LDS) and one 64-bit sort ranks them. Otherwise (n >
// 1024, or ties that leave more than 64 candidates) wave_topk_row ranks the
// row. n_load (>= n) entries of cand may be read; cand[i] is the score of
// block blk0 + i.
__device__ __forceinline__ uint64_t wave_topk_row_short(const float *cand, int n, int n_load,
                                                        int K, int lane, uint64_t *buf,
                                                        int blk0 = 0) {
    constexpr int kBatch = 16;
    if (n > 64 * kBatch) return wave_topk_row(cand, n, n_load, K, lane, buf, blk0);
    float v[kBatch];
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
        const int i = c * 64 + lane;
        v[c] = i < n_load && i < 64 * kBatch ? cand[i] : 0.f;
    }
    uint32_t o[kBatch];
    uint32_t lm = 0;
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
        const int i = c * 64 + lane;
        o[c] = i < n ? score_bits(v[c]) : 0u;
        lm = o[c] > lm ? o[c] : lm;
    }
    const uint32_t thr = (uint32_t)__shfl((int)wave_sort_desc_u32(lm, lane), K - 1);
    // Valid keys at or above the threshold: a per-lane count, then a wave
    // prefix sum from five ballots of the count bits (count <= 16).
    int my = 0;
#pragma unroll
    for (int c = 0; c < kBatch; ++c) my += (c * 64 + lane < n && o[c] >= thr) ? 1 : 0;
    const uint64_t below = (1ull << lane) - 1ull;
    int excl = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
        const uint64_t bm = __ballot((my >> bit) & 1);
        excl += __popcll(bm & below) << bit;
        total += __popcll(bm) << bit;
    }
    if (total > 64) return wave_topk_row(cand, n, n_load, K, lane, buf, blk0);
    int pos = excl;
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
        const int i = c * 64 + lane;
        if (i < n && o[c] >= thr) buf[pos++] = score_key(v[c], blk0 + i);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the list writes have landed
    __builtin_amdgcn_wave_barrier();
    const uint64_t x = wave_sort_desc(lane < total ? buf[lane] : 0, lane);
    __builtin_amdgcn_wave_barrier();
    return lane < K ? x : 0;
}

// Bitonic stages 2*RUN .. 64 over one key per lane, for lanes that already
// form runs of RUN keys with even runs descending and odd runs ascending (the
// state after stage RUN); ends descending, lane 0 the largest. RUN = 1 is a
// full sort.
template <int RUN>
__device__ __forceinline__ uint64_t bitonic_from_runs(uint64_t x, int lane) {
    if constexpr (RUN >= 64) return x;  // one run: already sorted
    if constexpr (RUN <= 1) x = bitonic_step<2, 1>(x, lane);
    if constexpr (RUN <= 2) {
        x = bitonic_step<4, 2>(x, lane);
        x = bitonic_step<4, 1>(x, lane);
    }
    if constexpr (RUN <= 4) {
        x = bitonic_step<8, 4>(x, lane);
        x = bitonic_step<8, 2>(x, lane);
        x = bitonic_step<8, 1>(x, lane);
    }
    if constexpr (RUN <= 8) {
        x = bitonic_step<16, 8>(x, lane);
        x = bitonic_step<16, 4>(x, lane);
        x = bitonic_step<16, 2>(x, lane);
        x = bitonic_step<16, 1>(x, lane);
    }
    if constexpr (RUN <= 16) {
        x = bitonic_step<32, 16>(x, lane);
        x = bitonic_step<32, 8>(x, lane);
        x = bitonic_step<32, 4>(x, lane);
        x = bitonic_step<32, 2>(x, lane);
        x = bitonic_step<32, 1>(x, lane);
    }
    x = bitonic_step<64, 32>(x, lane);
    x = bitonic_step<64, 16>(x, lane);
    x = bitonic_step<64, 8>(x, lane);
    x = bitonic_step<64, 4>(x, lane);
    x = bitonic_step<64, 2>(x, lane);
    return bitonic_step<64, 1>(x, lane);
}

// One 64-key register of the NW sorted runs of Kp keys in `runs` (register r
// holds keys r*64 .. r*64+63), loaded with odd runs reversed, then sorted.
template <int KP>
__device__ __forceinline__ uint64_t load_runs_sorted(const uint64_t *runs, int nkeys, int r,
                                                     int lane) {
    const int i = r * 64 + lane;
    const int pos = lane % KP, run0 = i - pos;
    const int j = ((lane / KP) & 1) ? run0 + KP - 1 - pos : i;
    const uint64_t x = i < nkeys ? runs[j] : 0;
    return bitonic_from_runs<KP>(x, lane);
}

// The NREG registers of runs (NW sorted runs of KP keys) merged pairwise into
// the 64 largest keys, descending.
template <int KP, int NREG>
__device__ __forceinline__ uint64_t merge_runs(const uint64_t *runs, int nkeys, int lane) {
    uint64_t r[NREG];
#pragma unroll
    for (int i = 0; i < NREG; ++i) r[i] = load_runs_sorted<KP>(runs, nkeys, i, lane);
#pragma unroll
    for (int step = 1; step < NREG; step *= 2)
#pragma unroll
        for (int i = 0; i + step < NREG; i += 2 * step)
            r[i] = merge_sorted_desc(r[i], r[i + step], lane);
    return r[0];
}

// Top-K (K <= 64) of one row by the NW (<= 16) waves of a workgroup: wave w
// ranks a contiguous share of the row's n pooled scores with
// wave_topk_row_short
// and writes its K best keys, zero-padded to Kp (the next power of two), to
// `runs` (LDS, NW * 64 keys); after a barrier wave 0 merges the NW sorted
// runs. `bufs` is NW * 64 keys of LDS (wave_topk_row's lists). Every thread of
// the workgroup must call it. Returns the K best keys, descending, in lanes
// 0..K-1 of wave 0; 0 in every other lane and wave. Up to n_load >= n scores
// may be read (see wave_topk_row).
template <int NW>
__device__ __forceinline__ uint64_t block_topk_row(const float *cand, int n, int n_load, int K,
                                                   int lane, int wave, uint64_t *bufs,
                                                   uint64_t *runs) {
    const int chunk = (n_load + NW - 1) / NW;
    const int b0 = wave * chunk;
    const int nw = min(max(n - b0, 0), chunk), nlw = min(max(n_load - b0, 0), chunk);
    const uint64_t mine = wave_topk_row_short(cand + b0, nw, nlw, K, lane, bufs + wave * 64, b0);
    const int kp = K <= 1 ? 1 : K <= 2 ? 2 : K <= 4 ? 4 : K <= 8 ? 8 : K <= 16 ? 16 : K <= 32 ? 32 : 64;
    if (lane < kp) runs[wave * kp + lane] = mine;  // lanes K..kp-1 hold 0
    __syncthreads();
    if (wave != 0) return 0;
    const int nkeys = NW * kp;
    // Up to 64 keys (Kp <= 8) are one register, sorted whole (runs of one).
    constexpr int R16 = (NW * 16 + 63) / 64, R32 = (NW * 32 + 63) / 64, R64 = NW;
    const uint64_t x = kp <= 8 ? merge_runs<1, 1>(runs, nkeys, lane)
                     : kp == 16 ? merge_runs<16, R16>(runs, nkeys, lane)
                     : kp == 32 ? merge_runs<32, R32>(runs, nkeys, lane)
                                : merge_runs<64, R64>(runs, nkeys, lane);
    return lane < K ? x : 0;
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

// Stream: nontemporal loads, for K/V rows that no other workgroup reads.
template <bool Stream>
__device__ __forceinline__ void load_chunk(ChunkRegs &cr, const bf16_t *kg_base,
                                           const bf16_t *vg_base, int tok0, int p, int lane) {
    const int col = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int tok = tok0 + rt * 16 + col;
        const bf16_t *kp = kg_base + (size_t)(tok <= p ? tok : p) * D + kg * 8;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) cr.kr[rt][kc] = Stream ? ld16_stream(kp + kc * 32) : ld16(kp + kc * 32);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int piece = lane + 64 * i;
        const int tok = tok0 + (piece >> 4);
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        const bf16_t *vp = vg_base + (size_t)tok * D + (piece & 15) * 8;
        cr.vr[i] = tok <= p ? (Stream ? ld16_stream(vp) : ld16(vp)) : z4;
    }
}

__device__ __forceinline__ void compute_chunk(WaveAttn &st, const bf16x8 (&qf)[4],
                                              const ChunkRegs &cr, int tok0, int p,
                                              float scale_log2, unsigned char *vrows, int lane);

// One 32-token chunk [tok0, tok0 + 32) of a kept block; keys past p are masked.
template <bool Stream = false>
__device__ __forceinline__ void attend_chunk(WaveAttn &st, const bf16x8 (&qf)[4],
                                             const bf16_t *kg_base, const bf16_t *vg_base,
                                             int tok0, int p, float scale_log2,
                                             unsigned char *vrows, int lane) {
    ChunkRegs cr;
    load_chunk<Stream>(cr, kg_base, vg_base, tok0, p, lane);
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

typedef __attribute__((ext_vector_type(4))) short v4i16;

__device__ __forceinline__ v4i16 pack_bf16x4(float a, float b, float c, float d) {
    const uint32_t lo = pack_bf16x2(a, b), hi = pack_bf16x2(c, d);
    return __builtin_bit_cast(v4i16, u32x2{lo, hi});
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

// A KV-major list entry: the row of the pass and the selection slot, as
// (row << kEntShift) | slot (slots < 64).
constexpr int kEntShift = 6;
constexpr int kEntMask = (1 << kEntShift) - 1;

__device__ __forceinline__ bool slot_kept(const int32_t *sel_row, int k, int n_valid) {
    const int blk = sel_row[k];
    if (blk < 0 || blk >= n_valid) return false;
    for (int k2 = 0; k2 < k; ++k2)
        if (sel_row[k2] == blk) return false;
    return true;
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
}  // namespace

#endif  // MSA_DEVICE_H

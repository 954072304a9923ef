// libmsa backward of the sparse branch for gfx950 (MI355X, CDNA4) and its
// entry point, msa_sparse_attn_backward.
#include <algorithm>
#include "msa_device.h"

namespace {

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
//                     batch's dS goes to LDS (two buffers, the second in the
//                     K staging area once each wave holds its K^T operands
//                     in registers), where dq^T = K^T dS^T over the block's
//                     128 keys, run after the next batch's products, gives
//                     tau * dq per (row, group, slot, head), bf16; one
//                     barrier per batch; an fp32 [dk; dv] partial per tile;
//   bwd_dkdv_reduce_kernel  per list: dk, dv = sum of its tiles' partials in
//                     tile order (added to the earlier passes' values);
//   bwd_dq_merge_kernel  dq of a (row, group) = fp32 sum of its kept slots'
//                     partials.
// delta comes first from bwd_delta_kernel. No floating-point atomics: every
// sum has one owner and a fixed order.

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
            const int64_t hrow =
                ((int64_t)b * T + t0 + (ent >> kEntShift)) * H + (int64_t)g * R + tc % R;
            l2 = lse[hrow] * kLog2e;
            dl = delta[hrow];
            pc = qs + t0 + (ent >> kEntShift);
            slot = (int)((((int64_t)b * rows + (ent >> kEntShift)) * ng + gl) * K +
                         (ent & kEntMask));
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
    // This wave's K^T operands of the dq product (d tiles 2*(w>>1) + i, all
    // 128 keys; keys 4*kg + 0..3 and 16 + 4*kg + 0..3 of each 32-key chunk),
    // read transposed from LDS once per tile. The K staging area then holds
    // the second dS buffer.
    bf16x8 kT[S / 32][2];
#pragma unroll
    for (int cc = 0; cc < S / 32; ++cc)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const unsigned char *p =
                k_s + (cc * 32 + 4 * kg + (col >> 2)) * kVRow + (2 * (wave >> 1) + i) * 32 + (col & 3) * 8;
            const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 16 * kVRow);
            kT[cc][i] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): k_s is read before it is reused
    auto ds_buf = [&](int i) -> unsigned char * { return i ? k_s : ds_s; };
    static_assert(S * kDsRow <= S * kVRow, "a dS buffer fits the K staging area");
    // dq^T = K^T dS^T of the batch at column cbq (its dS in dsb), tau applied:
    // wave w owns column tiles 2*(w&1) + j and d tiles 2*(w>>1) + i; dS^T is
    // read transposed from LDS in the K^T operands' key order.
    auto dq_batch = [&](int cbq, const unsigned char *dsb) {
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
                const unsigned char *p = dsb + krow * kDsRow + (2 * (wave & 1) + j) * 32 + (col & 3) * 8;
                const u32x2 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 16 * kDsRow);
                bq[j] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) dqa[i][j] = mfma16(kT[cc][i], bq[j], dqa[i][j]);
        }
        // Lane holds column 16*ct + col, d = 16*dt + 4*kg + r.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int tc = cbq + 16 * (2 * (wave & 1) + j) + col;
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
    };
    for (int cb = 0, cur = 0; cb < ncol; cb += kBwdCols, cur ^= 1) {
        // The other q / dout buffer was last read in the previous batch,
        // which ended with a barrier.
        if (cb + kBwdCols < ncol) {
            stage(cur ^ 1);
            if (cb + 2 * kBwdCols < ncol) fetch(cb + 2 * kBwdCols);
        }
        const unsigned char *q_s = q_buf[cur];
        const unsigned char *do_s = do_buf[cur];
        const float *b_lse2 = s_lse2 + cb;
        const float *b_dl = s_dl + cb;
        const int *b_pc = s_pc + cb;
        // P and dS of all four 16-column tiles first (their S and dP chains
        // are independent), then per pair of tiles one 16x16x32 product per d
        // tile whose k-slots 8*kg .. 8*kg+3 are columns 32*cp + 4*kg + 0..3
        // and slots 8*kg+4 .. 8*kg+7 columns 32*cp + 16 + 4*kg + 0..3 (the
        // same order in both operands).
        v4i16 pbA[kBwdCols / 32][2][KT], dsbA[kBwdCols / 32][2][KT];
#pragma unroll
        for (int cp = 0; cp < kBwdCols / 32; ++cp) {
            auto &pb = pbA[cp];
            auto &dsb = dsbA[cp];
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
                    *reinterpret_cast<v4i16 *>(ds_buf(cur) + (16 * (KT * wave + kt2) + col) * kDsRow +
                                               (16 * ct + 4 * kg) * 2) = dsb[hf][kt2];
                }
            }
        }
#pragma unroll
        for (int cp = 0; cp < kBwdCols / 32; ++cp) {
            auto &pb = pbA[cp];
            auto &dsb = dsbA[cp];
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
        // The previous batch's dq (its dS in the other buffer) overlaps this
        // batch's products across the waves; then one barrier: this batch's
        // dS is complete, the previous dS buffer and this q / dout buffer are
        // free, and the next batch is staged.
        if (cb > 0) dq_batch(cb - kBwdCols, ds_buf(cur ^ 1));
        __syncthreads();
    }
    if (ncol > 0) {
        const int last = (ncol - 1) / kBwdCols;
        dq_batch(last * kBwdCols, ds_buf(last & 1));
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
// summed in slot order; zero for a row outside the cache. The workgroup
// holds the R * D / 4 threads that sum, rounded up to whole waves.
__global__ __launch_bounds__(256) void bwd_dq_merge_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ kv_lens,
    const int32_t *__restrict__ q_start, const bf16_t *__restrict__ part_dq, int T, int G, int R,
    int Nmax, int K, int t0, int rows, int g0, int ng, float *__restrict__ dq) {
    __shared__ int32_t s_sel[KMAX];
    __shared__ int32_t s_kept[KMAX];
    __shared__ int32_t s_n;
    const int tid = threadIdx.x, lane = tid & 63, nthr = blockDim.x;
    const int64_t unit = blockIdx.x;
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
    const int H = G * R;
    for (int idx = tid; idx < R * (D / 4); idx += nthr) {
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

}  // namespace

extern "C" {

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
    // dq merge threads: R * D / 4 rounded up to whole waves, at most 256.
    const unsigned merge_threads = (unsigned)std::min(256, (R * (D / 4) + 63) / 64 * 64);
    for (int32_t g0 = 0; g0 < G; g0 += w.groups)
      for (int32_t t0 = 0; t0 < T; t0 += w.rows) {
        const int ng = w.groups;
        msa::build_pass_lists(w, base, sel, kv_lens, q_start, B, T, G, Nmax, K, t0, g0, st);
        bwd_tile_kernel<<<(unsigned)w.max_tiles, kBwdThreads, 0, st>>>(
            qp, kp, vp, kv_lens, q_start, lse, dop, delta, offsets, tile_first, tile_map, list,
            w.nlists, T, G, R, Nmax, K, t0, w.rows, g0, ng, w.nb_max, w.entries_per_tile, sl2,
            tau, part_dq, part_kv, reinterpret_cast<unsigned char *>(base + w.trash_off));
        bwd_dkdv_reduce_kernel<<<(unsigned)w.nlists, 256, 0, st>>>(
            tile_first, part_kv, G, Nmax, g0, ng, w.nb_max, tau, t0 > 0 ? 1 : 0, dk, dv);
        bwd_dq_merge_kernel<<<(unsigned)((int64_t)B * w.rows * ng), merge_threads, 0, st>>>(
            sel, kv_lens, q_start, part_dq, T, G, R, Nmax, K, t0, w.rows, g0, ng, dq);
        s = launch_status("sparse backward kernels");
        if (s != MSA_OK) return s;
    }
    return MSA_OK;
}

}  // extern "C"

// libmsa index projections for gfx950 (MI355X, CDNA4) and their entry point,
// msa_index_project.
//
// The index branch of the Tencent article ("Something BIG Is Coming
// 百万token上下文提速近10倍，MiniMax M3的稀疏注意力凭什么这么快", §二) forms one
// lightweight index query per GQA group from a token's hidden state, and the
// per-token index keys it scores against. Both are linear maps of the hidden
// state, so one GEMM produces them: C = hidden x W^T with W holding the G
// index-query projections and then the index-key projection, one output
// feature per row.
//
// Kernel:
//   idx_proj_kernel  one workgroup (eight waves) per (512 tokens, one
//                    128-feature head), the heads of a token tile back to
//                    back on one XCD. The K loop stages 32 hidden elements of
//                    the 128 W rows and of the 512 hidden rows per step by
//                    direct global->LDS loads into a ring of four stages
//                    (160 KiB; two steps in flight, one barrier per step);
//                    each wave computes 64 features of 128 tokens (a 2 x 4
//                    grid of 32x32x16 bf16 MFMA tiles, 128 fp32 accumulators
//                    per lane), W rows as the A operand so a lane ends with
//                    four consecutive features of one token; bf16 (nearest
//                    even) output. A step's staging loads and LDS operand
//                    reads are issued one by one between its MFMAs. Against
//                    256-token tiles of 64 x 64 per wave, the larger tiles
//                    read a quarter fewer operand bytes from LDS per MFMA,
//                    stage a sixth fewer bytes per flop and share each hidden
//                    row among five heads on one XCD over twice the tokens.
#include "msa_device.h"

namespace {

constexpr int kPjM = 512;            // tokens per workgroup
constexpr int kPjN = 128;            // output features per workgroup (= dI, one head)
constexpr int kPjK = 32;             // hidden elements per K step
constexpr int kPjRow = kPjK * 2;     // bytes of one staged row per step
constexpr int kPjStages = 4;         // staged K steps (ring)
constexpr int kPjWaveM = 128;                     // tokens per wave
constexpr int kPjWaveN = 64;                      // features per wave
constexpr int kPjWavesN = kPjN / kPjWaveN;        // waves across the features
constexpr int kPjWaves = kPjM / kPjWaveM * kPjWavesN;
constexpr int kPjTA = kPjWaveN / 32;              // 32-row W operand tiles per wave
constexpr int kPjOps = kPjTA + 4;                 // LDS operand reads per k-slice
constexpr int kPjProds = kPjTA * 4;               // MFMAs per k-slice
constexpr int kPjRunRows = 1024 / kPjRow;         // staged rows per 1 KiB run (16)
constexpr int kPjRunsW = kPjN / kPjRunRows;       // runs of the W tile (8)
constexpr int kPjRunsH = kPjM / kPjRunRows;       // of the hidden tile (32)
constexpr int kPjRunsPerWave = (kPjRunsW + kPjRunsH) / kPjWaves;  // 10
constexpr int kPjStage = (kPjRunsW + kPjRunsH) * 1024;            // bytes per stage
static_assert(kPjRunsPerWave * kPjWaves == kPjRunsW + kPjRunsH, "runs split evenly");
static_assert(kPjRunsW % kPjWaves == 0, "each wave's first runs are W runs");
static_assert(kPjProds >= kPjOps && kPjProds >= kPjRunsPerWave, "loads fit between products");

// Physical 16-byte slot of logical piece `piece` of staged row `row` (four
// pieces per 64-byte row, four rows per 256 bytes of banks): 16 lanes reading
// the same piece of 16 consecutive rows hit distinct banks.
__device__ __forceinline__ int pj_swz(int row, int piece) { return piece ^ ((row >> 2) & 3); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (LDS and export counters not waited on).
constexpr int pj_wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070 | 0x0F00; }
// The same with every LDS read of this wave done as well (lgkmcnt(0)).
constexpr int pj_wait_vm_lds(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

struct PjSlice {
    bf16x8 a[kPjTA], b[4];  // the wave's W rows 32t + j and hidden rows 32u + j
};

__global__ __launch_bounds__(kPjWaves * 64, 1) void idx_proj_kernel(
    const bf16_t *__restrict__ hidden, const bf16_t *__restrict__ w, int M, int Kh, int G,
    bf16_t *__restrict__ q_idx, bf16_t *__restrict__ k_idx) {
    // Ring of kPjStages K steps: [stage][W rows (8 KiB) | hidden rows (32 KiB)].
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kPjStages][kPjStage];
    // Workgroups are dealt to the eight XCDs in turn (id % 8); the G + 1 heads
    // of one 512-token tile run back to back on the same XCD, so the tile's
    // hidden rows are read from HBM about once and then from that XCD's L2.
    const int id = blockIdx.x;
    const int xcd = id % 8, s = id / 8;
    const int tile = (s / (G + 1)) * 8 + xcd;
    const int head = s % (G + 1);  // 0 .. G-1: index query of group `head`; G: index key
    const int64_t m0 = (int64_t)tile * kPjM;
    if (m0 >= M || (head == G && !k_idx)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = head * kPjN;
    const int j = lane & 31, half = lane >> 5;
    const int tw = wave / kPjWavesN * kPjWaveM;  // the wave's first token within the tile
    const int fw = wave % kPjWavesN * kPjWaveN;  // and its first feature
    // Stage hidden elements [k0, k0 + 32) of both operands: wave w loads runs
    // w, w + 8, ... (runs 0..7 the W tile, 8..39 the hidden tile); lane l
    // fills physical slot l & 3 of row 16*run' + l/4. Hidden rows past M load
    // row M - 1 (their results are not stored).
    auto stage_run = [&](int k0, int st, int i) {
        const int run = wave + kPjWaves * i;
        const bool is_w = i < kPjRunsW / kPjWaves;
        const int row = (is_w ? run : run - kPjRunsW) * kPjRunRows + (lane >> 2);
        const int piece = pj_swz(row, lane & 3);
        const bf16_t *src =
            is_w ? w + (size_t)(n0 + row) * Kh + k0 + piece * 8
                 : hidden + (size_t)min(m0 + row, (int64_t)M - 1) * Kh + k0 + piece * 8;
        __builtin_amdgcn_global_load_lds(
            (const void *)src, (__attribute__((address_space(3))) void *)(lds[st] + run * 1024),
            16, 0, 0);
    };
    auto stage = [&](int k0, int st) {
#pragma unroll
        for (int i = 0; i < kPjRunsPerWave; ++i) stage_run(k0, st, i);
    };
    // Lane (j, half) reads elements 16*ks + 8*half .. +7 of its rows; all of
    // its rows share j's swizzle (rows fw + 32t + j and tw + 32u + j differ
    // from j in multiples of 32), so one byte offset per k-slice serves every
    // read.
    int off[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) off[ks] = j * kPjRow + pj_swz(j, 2 * ks + half) * 16;
    // Operand r of a k-slice, in the order its products need them: a[0],
    // b[0..3], then the other a.
    auto read_op = [&](int st, int ks, PjSlice &o, int r) {
        const unsigned char *aw = lds[st] + fw * kPjRow + off[ks];
        const unsigned char *bh = lds[st] + kPjRunsW * 1024 + tw * kPjRow + off[ks];
        if (r == 0)
            o.a[0] = as_bf16x8(*reinterpret_cast<const u32x4 *>(aw));
        else if (r <= 4)
            o.b[r - 1] = as_bf16x8(*reinterpret_cast<const u32x4 *>(bh + 32 * (r - 1) * kPjRow));
        else
            o.a[r - 4] = as_bf16x8(*reinterpret_cast<const u32x4 *>(aw + 32 * (r - 4) * kPjRow));
    };
    auto read_slice = [&](int st, int ks, PjSlice &o) {
#pragma unroll
        for (int r = 0; r < kPjOps; ++r) read_op(st, ks, o, r);
    };
    f32x16 acc[kPjTA][4] = {};
    // nk >= 2 (the hidden size is a multiple of 64). Every step issues the
    // same loads, so one wait count serves all: the loads for steps past the
    // last reload the last step into the stage just freed, which no step
    // reads as data (the stale read of the last step below lands there too).
    const int nk = Kh / kPjK;
#pragma unroll
    for (int k = 0; k < kPjStages - 1; ++k) stage(min(k, nk - 1) * kPjK, k);
    // Step 0 complete for every wave, then its first k-slice into registers.
    __builtin_amdgcn_s_waitcnt(pj_wait_vm(2 * kPjRunsPerWave));
    __builtin_amdgcn_s_barrier();
    PjSlice s0, s1;
    read_slice(0, 0, s0);
    for (int kb = 0; kb < nk; ++kb) {
        // Step kb + 1 complete for every wave (its first k-slice is read at
        // the end of this step): this wave's loads of it have landed (only
        // those of step kb + 2 may still be in flight), then the barrier. No
        // wave still reads the stage of step kb - 1 (every read of it fed an
        // MFMA issued before the barrier), so step kb + 3 may refill it. The
        // first k-slice of step kb, read during the previous step, is in
        // registers by now; waiting for it here leaves the products below
        // waiting only on reads issued several MFMAs before them.
        __builtin_amdgcn_s_waitcnt(pj_wait_vm_lds(kPjRunsPerWave));
        __builtin_amdgcn_s_barrier();
        // The order below is fixed (nothing is scheduled across the fences):
        // the step's staging loads and the reads of its second k-slice go out
        // one by one between the first k-slice's products, and the reads of
        // the next step's first k-slice between the second's, so the MFMA
        // pipe is not left idle while they issue. (On the last step that
        // read is of a stale stage, in bounds and unused.)
        const int st = kb % kPjStages, st_next = (kb + 1) % kPjStages;
        const int k_stage = min(kb + kPjStages - 1, nk - 1) * kPjK;
        const int st_stage = (kb + kPjStages - 1) % kPjStages;
#pragma unroll
        for (int i = 0; i < kPjProds; ++i) {
            acc[i >> 2][i & 3] = mfma32(s0.a[i >> 2], s0.b[i & 3], acc[i >> 2][i & 3]);
            if (i < kPjRunsPerWave) stage_run(k_stage, st_stage, i);
            if (i < kPjOps) read_op(st, 1, s1, i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < kPjProds; ++i) {
            acc[i >> 2][i & 3] = mfma32(s1.a[i >> 2], s1.b[i & 3], acc[i >> 2][i & 3]);
            if (i < kPjOps) read_op(st_next, 0, s0, i);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // The trailing reloads write LDS: they land before the workgroup ends.
    __builtin_amdgcn_s_waitcnt(pj_wait_vm(0));
    // acc[t][u] lane l: token tw + 32u + (l & 31), features
    // fw + 32t + 8*(i>>2) + 4*(l>>5) + (i&3): four consecutive features per
    // group of four values, stored as 8 bytes.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t m = m0 + tw + 32 * u + j;
        if (m >= M) continue;
        bf16_t *dst = head < G ? q_idx + ((size_t)m * G + head) * kPjN : k_idx + (size_t)m * kPjN;
#pragma unroll
        for (int t = 0; t < kPjTA; ++t)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int f = fw + 32 * t + 8 * i4 + 4 * half;
                *reinterpret_cast<u32x2 *>(dst + f) =
                    u32x2{pack_bf16x2(acc[t][u][4 * i4], acc[t][u][4 * i4 + 1]),
                          pack_bf16x2(acc[t][u][4 * i4 + 2], acc[t][u][4 * i4 + 3])};
            }
    }
}

}  // namespace

extern "C" {

msa_status msa_index_project(const msa_config *cfg, int32_t M, int32_t hidden_dim,
                             const void *hidden, const void *w, void *q_idx, void *k_idx,
                             void *stream) {
    msa::clear_error();
    msa_status s = msa::check_project_args(cfg, M, hidden_dim, hidden, w, q_idx, k_idx);
    if (s != MSA_OK || M == 0) return s;
    const int G = cfg->num_kv_groups;
    const int64_t tiles8 = ((int64_t)(M + kPjM - 1) / kPjM + 7) / 8 * 8;
    if (tiles8 * (G + 1) > 0x7FFFFFFF)
        return msa::fail(MSA_ERR_UNSUPPORTED, "too many index projection tiles for one launch");
    idx_proj_kernel<<<(unsigned)(tiles8 * (G + 1)), kPjWaves * 64, 0,
                      reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const bf16_t *>(hidden), static_cast<const bf16_t *>(w), M, hidden_dim, G,
        static_cast<bf16_t *>(q_idx), static_cast<bf16_t *>(k_idx));
    return launch_status("index projection kernel");
}

}  // extern "C"

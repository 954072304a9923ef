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
//   idx_proj_kernel  one workgroup per (256 tokens, one 128-feature head),
//                    the heads of a token tile back to back on one XCD:
//                    the K loop stages 64 hidden elements of the 128 W rows
//                    and of the 256 hidden rows per step by direct
//                    global->LDS loads into a ring of three stages (two
//                    steps in flight, one barrier per step); eight waves
//                    each compute a 64 x 64 tile with
//                    32x32x16 bf16 MFMA (W rows as the A operand, so a lane
//                    ends with four consecutive features of one token), fp32
//                    accumulation, bf16 (nearest even) output.
#include "msa_device.h"

namespace {

constexpr int kPjM = 256;            // tokens per workgroup
constexpr int kPjN = 128;            // output features per workgroup (= dI, one head)
constexpr int kPjK = 64;             // hidden elements per K step
constexpr int kPjRow = kPjK * 2;     // bytes of one staged row per step
constexpr int kPjStages = 3;         // staged K steps in flight (ring)
constexpr int kPjWaves = 8;
constexpr int kPjRunsW = kPjN * kPjRow / 1024;    // 1 KiB runs of the W tile (16)
constexpr int kPjRunsH = kPjM * kPjRow / 1024;    // of the hidden tile (32)
constexpr int kPjRunsPerWave = (kPjRunsW + kPjRunsH) / kPjWaves;  // 6
constexpr int kPjStage = (kPjRunsW + kPjRunsH) * 1024;            // bytes per stage

// Physical 16-byte slot of logical piece `piece` of staged row `row` (eight
// pieces per 128-byte row, two rows per 256 bytes of banks): 16 lanes reading
// the same piece of 16 consecutive rows hit distinct banks.
__device__ __forceinline__ int pj_swz(int row, int piece) { return piece ^ ((row >> 1) & 7); }

__global__ __launch_bounds__(kPjWaves * 64, 1) void idx_proj_kernel(
    const bf16_t *__restrict__ hidden, const bf16_t *__restrict__ w, int M, int Kh, int G,
    bf16_t *__restrict__ q_idx, bf16_t *__restrict__ k_idx) {
    // Ring of kPjStages K steps: [stage][W rows (16 KiB) | hidden rows (32 KiB)].
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kPjStages][kPjStage];
    // Workgroups are dealt to the eight XCDs in turn (id % 8); the G + 1 heads
    // of one 256-token tile run back to back on the same XCD, so the tile's
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
    const int fw = (wave & 1) * 64, tw = (wave >> 1) * 64;  // the wave's features and tokens
    // Stage hidden elements [k0, k0 + 64) of both operands: wave w loads runs
    // w, w + 8, ... (runs 0..15 the W tile, 16..47 the hidden tile); lane l
    // fills physical slot l & 7 of row 8*run' + l/8. Hidden rows past M load
    // row M - 1 (their results are not stored).
    auto stage = [&](int k0, int st) {
#pragma unroll
        for (int i = 0; i < kPjRunsPerWave; ++i) {
            const int run = wave + kPjWaves * i;
            const bool is_w = run < kPjRunsW;
            const int row = (is_w ? run : run - kPjRunsW) * 8 + (lane >> 3);
            const int piece = pj_swz(row, lane & 7);
            const bf16_t *src =
                is_w ? w + (size_t)(n0 + row) * Kh + k0 + piece * 8
                     : hidden + (size_t)min(m0 + row, (int64_t)M - 1) * Kh + k0 + piece * 8;
            __builtin_amdgcn_global_load_lds(
                (const void *)src, (__attribute__((address_space(3))) void *)(lds[st] + run * 1024),
                16, 0, 0);
        }
    };
    f32x16 acc[2][2] = {};
    const int nk = Kh / kPjK;
#pragma unroll
    for (int k = 0; k < kPjStages - 1; ++k)
        if (k < nk) stage(k * kPjK, k);
    for (int kb = 0; kb < nk; ++kb) {
        // This wave's loads of step kb have landed (only the next step's
        // kPjRunsPerWave loads may still be in flight) and its LDS reads of
        // step kb - 1 are done; after the barrier every wave's have, so step kb
        // is complete and the stage of step kb - 1 is free for step kb + 2.
        if (kb + 1 < nk)
            __builtin_amdgcn_s_waitcnt(0x0070 | kPjRunsPerWave);  // vmcnt(6) lgkmcnt(0)
        else
            __builtin_amdgcn_s_waitcnt(0x0070);                    // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (kb + kPjStages - 1 < nk)
            stage((kb + kPjStages - 1) * kPjK, (kb + kPjStages - 1) % kPjStages);
        const unsigned char *aw = lds[kb % kPjStages];
        const unsigned char *bh = aw + kPjRunsW * 1024;
        // All of the step's operands first (lane (j, half) holds elements
        // 16*ks + 8*half .. +7 of its row), then the 16 products.
        bf16x8 a[4][2], bt[4][2];
#pragma unroll
        for (int ks = 0; ks < kPjK / 16; ++ks) {
            const int p = 2 * ks + half;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ra = fw + 32 * t + j, rb = tw + 32 * t + j;
                a[ks][t] = as_bf16x8(*reinterpret_cast<const u32x4 *>(aw + ra * kPjRow + pj_swz(ra, p) * 16));
                bt[ks][t] = as_bf16x8(*reinterpret_cast<const u32x4 *>(bh + rb * kPjRow + pj_swz(rb, p) * 16));
            }
        }
#pragma unroll
        for (int ks = 0; ks < kPjK / 16; ++ks)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u) acc[t][u] = mfma32(a[ks][t], bt[ks][u], acc[t][u]);
        // Interleave: the first step's four operand reads, then one MFMA per
        // read of the next steps' operands.
#pragma unroll
        for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    // acc[t][u] lane l: token tw + 32u + (l & 31), features
    // fw + 32t + 8*(i>>2) + 4*(l>>5) + (i&3): four consecutive features per
    // group of four values, stored as 8 bytes.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t m = m0 + tw + 32 * u + j;
        if (m >= M) continue;
        bf16_t *dst = head < G ? q_idx + ((size_t)m * G + head) * kPjN : k_idx + (size_t)m * kPjN;
#pragma unroll
        for (int t = 0; t < 2; ++t)
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

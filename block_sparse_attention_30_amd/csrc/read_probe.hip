// Ceiling probes for the benchmark, to set beside the published peaks:
//   - a streaming read of a device buffer (plain or nontemporal loads), the
//     HBM read bandwidth a kernel that only loads can reach on this GPU;
//   - a streaming copy between two device buffers (plain or nontemporal
//     stores), the bandwidth of an even mix of reads and writes;
//   - a loop of independent MFMAs (32x32x16 bf16 or 32x32x64 OCP E4M3) with
//     no memory traffic, the matrix throughput a kernel can sustain at the
//     clock the chip holds under that load.
// Not part of the MSA library: built into its own shared object and loaded
// by the benchmark only.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w reads 16-byte words [w * per_wg, (w + 1) * per_wg), eight loads
// per thread in flight, plain or nontemporal loads; a value is written only if
// the xor of everything read equals a marker, so the loads are kept but
// nothing is stored in practice.
template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p,
                                                          size_t per_wg, unsigned *sink) {
    constexpr int U = 8;
    const u32x4 *base = p + (size_t)blockIdx.x * per_wg;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t i = threadIdx.x; i < per_wg; i += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t j = i + (size_t)u * 256;
            if (j < per_wg) v[u] = NT ? __builtin_nontemporal_load(base + j) : base[j];
            else v[u] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    const unsigned r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (r == 0x9E3779B9u) sink[blockIdx.x] = r;
}

// Workgroup w copies 16-byte words [w * per_wg, (w + 1) * per_wg) of src to
// dst, eight loads per thread in flight, plain or nontemporal stores.
template <bool NT>
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4 *__restrict__ src,
                                                          u32x4 *__restrict__ dst, size_t per_wg) {
    constexpr int U = 8;
    const size_t base = (size_t)blockIdx.x * per_wg;
    for (size_t i = threadIdx.x; i < per_wg; i += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t j = i + (size_t)u * 256;
            if (j < per_wg) v[u] = src[base + j];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t j = i + (size_t)u * 256;
            if (j < per_wg) {
                if (NT)
                    __builtin_nontemporal_store(v[u], dst + base + j);
                else
                    dst[base + j] = v[u];
            }
        }
    }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Every wave runs `iters` rounds of kAcc independent MFMAs (no operand
// traffic: A and B stay in registers); the accumulators are summed and
// written only if they equal a marker, so the products are kept.
constexpr int kAcc = 4;

template <bool F8>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, unsigned *sink) {
    f32x16 acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    const unsigned t = threadIdx.x;
    if constexpr (F8) {
        // E4M3 bytes 0x30..0x3F: values in [0.5, 1) and [1, 2), no NaN.
        const int byte = 0x30 | (int)(t & 15);
        const int w = byte | (byte << 8) | (byte << 16) | (byte << 24);
        const i32x8 a = {w, w, w, w, w, w, w, w};
        const i32x8 b = {w ^ 0x01010101, w, w, w, w, w, w, w ^ 0x02020202};
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < kAcc; ++j)
                acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0,
                                                                         127, 0, 127);
        }
    } else {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)(1.0f + (float)((t + e) & 7) * 0.125f);
            b[e] = (__bf16)(0.5f - (float)((t ^ e) & 3) * 0.0625f);
        }
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < kAcc; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    if (s == 1.2345f) sink[blockIdx.x] = 1u;
}

}  // namespace

extern "C" {

// Runs the MFMA loop (fp8 != 0: 32x32x64 E4M3 with unit scales; else
// 32x32x16 bf16) on `wgs` workgroups of four waves, `iters` rounds of four
// MFMAs per wave, on `stream`; `sink` holds at least `wgs` uint32. Writes the
// products' flop count (2*M*N*K per MFMA) to *flops. Returns 0, -1 on bad
// arguments, or the HIP error code of the launch.
int msa_probe_mfma(int fp8, int wgs, int iters, void *sink, double *flops, void *stream) {
    if (!sink || !flops || wgs <= 0 || iters <= 0) return -1;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const double per = fp8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
    *flops = per * kAcc * (double)iters * 4.0 * (double)wgs;
    if (fp8)
        mfma_loop_kernel<true><<<(unsigned)wgs, 256, 0, st>>>(iters, static_cast<unsigned *>(sink));
    else
        mfma_loop_kernel<false><<<(unsigned)wgs, 256, 0, st>>>(iters, static_cast<unsigned *>(sink));
    return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16 * wgs) from `src` to `dst` with `wgs`
// workgroups on `stream`, with nontemporal stores if `nontemporal` is nonzero.
// Returns 0, or -1 on bad arguments, or the HIP error code of the launch.
int msa_probe_stream_copy(const void *src, void *dst, size_t bytes, int wgs, int nontemporal,
                          void *stream) {
    if (!src || !dst || wgs <= 0 || bytes == 0 || bytes % (16 * (size_t)wgs) != 0) return -1;
    const size_t per_wg = bytes / 16 / (size_t)wgs;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (nontemporal)
        stream_copy_kernel<true><<<(unsigned)wgs, 256, 0, st>>>(
            static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), per_wg);
    else
        stream_copy_kernel<false><<<(unsigned)wgs, 256, 0, st>>>(
            static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), per_wg);
    return (int)hipGetLastError();
}

// Reads `bytes` of `buf` (a multiple of 16 * wgs) with `wgs` workgroups on
// `stream`, with nontemporal loads if `nontemporal` is nonzero; `sink` holds
// at least `wgs` uint32. Returns 0, or -1 on bad arguments, or the HIP error
// code of the launch.
int msa_probe_stream_read(const void *buf, size_t bytes, int wgs, int nontemporal, void *sink,
                          void *stream) {
    if (!buf || !sink || wgs <= 0 || bytes == 0 || bytes % (16 * (size_t)wgs) != 0) return -1;
    const size_t per_wg = bytes / 16 / (size_t)wgs;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (nontemporal)
        stream_read_kernel<true><<<(unsigned)wgs, 256, 0, st>>>(
            static_cast<const u32x4 *>(buf), per_wg, static_cast<unsigned *>(sink));
    else
        stream_read_kernel<false><<<(unsigned)wgs, 256, 0, st>>>(
            static_cast<const u32x4 *>(buf), per_wg, static_cast<unsigned *>(sink));
    return (int)hipGetLastError();
}

}  // extern "C"

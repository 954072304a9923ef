// A streaming read of a device buffer (plain or nontemporal loads), for the
// benchmark's measured HBM read ceiling (the bandwidth a kernel that only loads can reach on this
// GPU, to set beside the published peak). Not part of the MSA library: it is
// built into its own shared object and loaded by the benchmark only.
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

}  // namespace

extern "C" {

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

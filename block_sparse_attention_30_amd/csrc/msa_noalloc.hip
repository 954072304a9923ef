// msa_decode_no_alloc: the decode step of msa_decode with its scratch memory
// (pooled block scores, split partials, arrival counters) in a fixed device
// array of the library instead of a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation). Same kernels as msa_decode.
//
// The array lives in the library's code object; every GPU the library runs
// on holds its own copy, at its own address, until the process ends. Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the device symbol): the first call on a device looks up that
// device's address with hipGetSymbolAddress and keeps it.
#include <mutex>

#include "msa_device.h"

namespace {

// Largest scratch one call may use: 32 MiB holds, for example, the 16 x 131072
// and the 4 x 1048576 decode batches (G = 4, R = 8, K = 16) with room to spare.
constexpr size_t kScratchBytes = (size_t)32 << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The address of `scratch` on the current device, looked up on the first call
// on that device (with it current) and kept.
msa_status scratch_of_current_device(char **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return msa::fail(MSA_ERR_HIP, "hipGetDevice: %s (%s)", hipGetErrorName(e),
                         hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return msa::fail(MSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return msa::fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s (%s)",
                             dev, hipGetErrorName(e), hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<char *>(g_scratch_ptr[dev]);
    return MSA_OK;
}

}  // namespace

extern "C" {

size_t msa_decode_no_alloc_max_scratch(void) { return kScratchBytes; }

msa_status msa_decode_no_alloc(const msa_config *cfg, int32_t B, int32_t Nmax, const void *q,
                               const void *q_idx, const void *k_idx, const void *k_cache,
                               const void *v_cache, const int32_t *kv_lens, int32_t *sel,
                               float *sel_scores, void *out, float *lse, void *stream) {
    msa::clear_error();
    msa_status s = msa::check_decode_shapes(cfg, B, Nmax, q, q_idx, k_idx, k_cache, v_cache,
                                            kv_lens, sel, sel_scores, out, lse);
    if (s != MSA_OK || B == 0) return s;
    const size_t need = msa::decode_ws(cfg, B, Nmax, true).total;
    if (need > kScratchBytes)
        return msa::fail(MSA_ERR_WORKSPACE,
                         "msa_decode_no_alloc: these shapes need %zu bytes of scratch, more than "
                         "its fixed %zu (call msa_decode with a workspace instead)",
                         need, kScratchBytes);
    char *base = nullptr;
    if ((s = scratch_of_current_device(&base)) != MSA_OK) return s;
    return msa::decode_step(cfg, B, Nmax, q, q_idx, k_idx, k_cache, v_cache, kv_lens, sel,
                            sel_scores, out, lse, base, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

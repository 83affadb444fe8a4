// specverify_noalloc.hip -- spec_verify for callers that cannot allocate:
// its scratch lives in a fixed device array instead of a caller workspace.
//
// The array is a file-scope __device__ variable, so every GPU the library runs
// on holds its own copy (kScratchBytes) from the first use until the process
// ends.  Host code never passes the array's name to a kernel (on the host that
// name is only a stand-in): once per device, with that device current, the
// device address is looked up with hipGetSymbolAddress and kept, and that
// address is what spec_verify's kernels receive as their workspace.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "specverify.h"

namespace {

constexpr size_t kScratchBytes = SPEC_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's copy of the scratch array (nullptr on failure).
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" spec_status spec_verify_noalloc(const void *target, const void *draft,
                                           const int32_t *draft_tokens, const int32_t *kept_len,
                                           const void *draft_stats, uint64_t seed, int32_t mode,
                                           const spec_params *params, const spec_verify_out *out,
                                           void *stream) {
    const size_t need = spec_workspace_bytes(params);
    if (need > kScratchBytes) return SPEC_ERR_UNSUPPORTED;  // beyond the fixed scratch
    if (need == 0 || (params && params->batch == 0))  // invalid or empty: spec_verify says which
        return spec_verify(target, draft, draft_tokens, kept_len, draft_stats, seed, mode, params,
                           out, nullptr, 0, stream);
    void *ws = device_scratch();
    if (!ws) return SPEC_ERR_HIP;
    return spec_verify(target, draft, draft_tokens, kept_len, draft_stats, seed, mode, params, out,
                       ws, kScratchBytes, stream);
}

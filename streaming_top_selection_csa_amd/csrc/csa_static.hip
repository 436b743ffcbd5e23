// csa_static.hip -- csa_index_static: csa_index_ex with its scratch in a
// fixed device array instead of caller or library allocations, for callers
// that cannot allocate device memory (code under graph capture, tight
// serving loops, hosts that forbid allocation).
//
// The array `scratch` below lives in the code object: every GPU the library
// is loaded on holds its own copy until the process ends.  Host code never
// uses the array's name as an address (in host code it is only a stand-in
// for the device symbol); it asks the runtime for the device address once
// per device and passes that pointer to the kernels as their workspace.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "csa_index.h"

namespace {

constexpr size_t kScratchBytes = CSA_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void *g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device.  Returns CSA_OK or CSA_ERR_HIP.
int scratch_ptr(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA_ERR_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return CSA_OK;
}

}  // namespace

extern "C" int csa_index_static(const void *q, const float *w, const void *k_cmp,
                                const csa_desc *desc, int32_t m, int32_t k, int32_t *out_idx,
                                float *out_score, const csa_options *opt, hipStream_t stream)
{
    csa_options o{};
    if (opt) o = *opt;
    if (o.workspace || o.workspace_bytes) return CSA_ERR_INVALID_ARG;
    if (!out_score) o.flags |= CSA_FLAG_NO_SCORE;
    csa_plan_info info{};
    int rc = csa_plan_query(desc, m, k, &o, &info);
    if (rc != CSA_OK) return rc;
    // an automatic partition size shrinks until the candidate logs fit
    if (info.workspace_bytes > kScratchBytes && o.chunk_keys == 0) {
        for (int c = info.chunk_keys / 2; c >= 64 && info.workspace_bytes > kScratchBytes; c /= 2) {
            o.chunk_keys = c;
            rc = csa_plan_query(desc, m, k, &o, &info);
            if (rc != CSA_OK) return rc;
        }
    }
    if (info.workspace_bytes > kScratchBytes) return CSA_ERR_WORKSPACE;
    void *ws = nullptr;
    rc = scratch_ptr(&ws);
    if (rc != CSA_OK) return rc;
    o.workspace = ws;
    o.workspace_bytes = kScratchBytes;
    return csa_index_ex(q, w, k_cmp, desc, m, k, out_idx, out_score, &o, stream);
}

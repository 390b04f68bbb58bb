// attn_fwd_noalloc: attn_fwd for callers that cannot allocate device memory.
// The key-split workspace (the per-row, per-range (m, l, o) records that the
// merge kernel reads) lives in a static device array of this file, one copy
// per GPU, instead of a buffer the caller passes in.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace {

static_assert(ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// The workspace of attn_fwd_noalloc. In host code `scratch` names a host-side
// stand-in, not device memory: only the address hipGetSymbolAddress returns
// for the current device may reach a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, once known

// Device address of `scratch` on device `dev`, looked up once per device
// with that device current (each GPU holds its own copy of the array).
int scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return ATTN_E_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return ATTN_E_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_E_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return ATTN_E_HIP;
        if (e != hipSuccess || p == nullptr) return ATTN_E_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Sq, int Sk, int d, float scale, int causal,
                                int layout, int dtype, const int32_t* kv_len, void* stream) {
    int rc = attn::check_fwd_call(q, k, v, o, lse, B, H, Sq, Sk, d, scale, layout, dtype, kv_len);
    if (rc != ATTN_OK) return rc;
    const size_t need = attn_fwd_workspace_size(B, H, Sq, Sk, d, dtype, causal);
    if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_E_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0) {
        // the device the stream belongs to (the null stream: the current one)
        int dev = -1;
        const hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                               : hipGetDevice(&dev);
        if (e != hipSuccess) return ATTN_E_HIP;
        rc = scratch_address(dev, &ws);
        if (rc != ATTN_OK) return rc;
    }
    // Every record the merge reads is written earlier in the same call, so
    // nothing needs clearing between calls.
    return attn_fwd(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, layout, dtype, kv_len, ws,
                    need > 0 ? (size_t)ATTN_NOALLOC_SCRATCH_BYTES : 0, stream);
}

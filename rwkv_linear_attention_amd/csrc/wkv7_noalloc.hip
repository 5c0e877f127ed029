// Allocation-free variant of wkv7_bwd for callers that cannot allocate
// device memory (code under HIP graph capture, tight training loops,
// harnesses that forbid hipMalloc).  The backward's workspace (state
// checkpoints, and the per-sequence gradients of a shared initial state)
// lives in a fixed device array of this file instead of a caller buffer;
// everything else is wkv7_bwd, kernels included.
#include <stdint.h>

#include <mutex>

#include "../../include/wkv7.h"
#include "wkv7_internal.hpp"

namespace {

// One array per GPU the library runs on, held until the process ends.
constexpr size_t kScratchBytes = WKV7_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current.  The name `scratch` in host code is only a host-side
// stand-in for the symbol and is never passed to a kernel or a copy.
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

wkv7_status_t scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WKV7_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WKV7_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return WKV7_OK;
}

}  // namespace

extern "C" {

wkv7_status_t wkv7_bwd_noalloc(int dtype, int B, int T, int H, int K, int V,
                               const void *r, const void *w, const void *k,
                               const void *v, const void *a, const void *b,
                               const float *initial_state, int n_state, const uint8_t *mask,
                               const void *d_o, const float *d_final_state,
                               void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                               float *d_initial_state, void *stream)
{
    // Every argument is checked on the host before any HIP call: wkv7_bwd's
    // own checks, then the scratch bound.
    const wkv7_status_t st = (wkv7_status_t)wkv7::check_bwd_args(
        dtype, B, T, H, K, V, r, w, k, v, a, b, initial_state, n_state, d_o, d_final_state, dr, dw, dk, dv, da, db,
        d_initial_state);
    if (st != WKV7_OK) return st;
    if (wkv7::bwd_workspace_bytes(B, T, H, K) > kScratchBytes) return WKV7_ERR_TOO_LARGE;
    void *ws = nullptr;
    if (T > 0) {
        const wkv7_status_t sst = scratch_of_current_device(&ws);
        if (sst != WKV7_OK) return sst;
    }
    return wkv7_bwd(dtype, B, T, H, K, V, r, w, k, v, a, b, initial_state, n_state, mask, d_o, d_final_state,
                    dr, dw, dk, dv, da, db, d_initial_state, ws, ws ? kScratchBytes : 0, stream);
}

}  // extern "C"

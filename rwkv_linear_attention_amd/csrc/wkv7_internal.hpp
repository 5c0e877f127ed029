// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

struct FwdArgs {
    int B, T, H, D;                      // D = K = V
    const void *r, *w, *k, *v, *a, *b;   // [B,T,H,D], I/O dtype
    const float *s0;                     // [B,H,D,D] or nullptr
    const uint8_t *mask;                 // [B,T] or nullptr
    void *o;                             // [B,T,H,D], I/O dtype
    float *sf;                           // [B,H,D,D] or nullptr
};

struct StepArgs {
    int B, H, D;
    const void *r, *w, *k, *v, *a, *b;   // [B,H,D]
    float *state;                        // [B,H,D,D], in place
    void *o;                             // [B,H,D]
};

// dtype: 0 = fp32, 1 = bf16 (values of wkv7_dtype_t).
hipError_t launch_recurrent(int dtype, const FwdArgs &args, hipStream_t stream);
hipError_t launch_chunked(const FwdArgs &args, hipStream_t stream);     // bf16 only
hipError_t launch_step(int dtype, const StepArgs &args, hipStream_t stream);
// final_state = initial_state (or zeros) for T == 0.
hipError_t launch_state_copy(const float *s0, float *sf, size_t n, hipStream_t stream);

}  // namespace wkv7

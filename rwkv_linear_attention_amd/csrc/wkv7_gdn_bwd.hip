// Backward of the Gated DeltaNet forward (rwkv-ops README, sections
// "gdn_recurrent 使用方法" and "gdn_chunk 使用方法": the training entries take
// q, k [B,T,H,K] normalised inside, v [B,T,H,V], a log-space gate g [B,T,H],
// a write strength beta [B,T,H] and an optional initial state [B,H,K,V] or
// [1,H,K,V], and backpropagate).
//
// The gated delta rule is the generalized rule for the operands r = qn,
// w = g, k = beta kn, a = -e^g beta kn, b = kn, so the two backward launches
// of wkv7_backward.hip run in their Gated DeltaNet mode: they form those
// operands from q, k, g and beta while staging each chunk, and apply the
// chain rule back to q, k, g and beta when storing the token gradients.  This
// file adds only the handling of one shared initial state ([1,H,K,V] with
// B > 1): it is copied to one row per sequence before the backward, and its
// gradient is the sum over the sequences, taken in sequence order afterwards
// (no atomics, so the result is deterministic).
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace wkv7 {
namespace {

// dst[b] = src (one [H,D,D] state copied to each of the B sequences).
__global__ __launch_bounds__(256) void expand_state_kernel(const float *__restrict__ src, float *__restrict__ dst,
                                                           size_t per, int B)
{
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= per) return;
    const f32x4 x = *(const f32x4 *)(src + i);
    for (int b = 0; b < B; ++b) *(f32x4 *)(dst + (size_t)b * per + i) = x;
}

// dst = sum over b of src[b], in order b = 0 .. B-1 (src == nullptr: zeros).
__global__ __launch_bounds__(256) void sum_states_kernel(const float *__restrict__ src, float *__restrict__ dst,
                                                         size_t per, int B)
{
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= per) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (src)
        for (int b = 0; b < B; ++b) acc += *(const f32x4 *)(src + (size_t)b * per + i);
    *(f32x4 *)(dst + i) = acc;
}

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

size_t gdn_bwd_workspace_bytes(int B, int T, int H, int D)
{
    return 2 * up((size_t)B * H * D * D * sizeof(float)) + bwd_workspace_bytes(B, T, H, D);
}

hipError_t launch_gdn_backward(int dtype, const GdnBwdArgs &p, hipStream_t stream)
{
    const size_t per_state = (size_t)p.H * p.D * p.D, states = up((size_t)p.B * per_state * sizeof(float));
    char *ws = (char *)p.ws;
    float *s0x = (float *)ws;                 // the shared initial state, one row per sequence
    float *ds0x = (float *)(ws + states);     // per-sequence initial-state gradients
    void *wkv_ws = ws + 2 * states;
    const unsigned grid_state = (unsigned)((per_state / 4 + 255) / 256);
    const bool shared = p.s0 && p.n_state == 1 && p.B > 1;
    hipError_t e = hipSuccess;
    const float *s0 = p.s0;
    if (shared) {
        hipLaunchKernelGGL(expand_state_kernel, dim3(grid_state), dim3(256), 0, stream, p.s0, s0x, per_state, p.B);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        s0 = s0x;
    }
    float *d_s0 = p.d_s0 ? (shared ? ds0x : p.d_s0) : nullptr;
    BwdArgs wa{p.B, p.T, p.H, p.D, p.q, p.g, p.k, p.v, p.beta, nullptr, s0, nullptr, p.d_o, p.d_sf,
               p.dq, p.dg, p.dk, p.dv, p.dbeta, nullptr, d_s0, wkv_ws};
    wa.gdn = true;
    if ((e = launch_backward(dtype, wa, stream)) != hipSuccess) return e;
    if (shared && p.d_s0) {
        hipLaunchKernelGGL(sum_states_kernel, dim3(grid_state), dim3(256), 0, stream, ds0x, p.d_s0, per_state, p.B);
        e = hipGetLastError();
    }
    return e;
}

// T == 0 with a shared initial state: its gradient is the sum of the B
// final-state gradients (zeros without them).
hipError_t launch_state_sum(const float *src, float *dst, int B, size_t per, hipStream_t stream)
{
    hipLaunchKernelGGL(sum_states_kernel, dim3((unsigned)((per / 4 + 255) / 256)), dim3(256), 0, stream, src, dst,
                       per, B);
    return hipGetLastError();
}

}  // namespace wkv7

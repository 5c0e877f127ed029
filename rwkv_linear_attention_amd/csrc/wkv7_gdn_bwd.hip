// Backward of the Gated DeltaNet forward (rwkv-ops README, sections
// "gdn_recurrent 使用方法" and "gdn_chunk 使用方法": the training entries take
// q, k [B,T,H,K] normalised inside, v [B,T,H,V], a log-space gate g [B,T,H],
// a write strength beta [B,T,H] and an optional initial state [B,H,K,V] or
// [1,H,K,V], and backpropagate).
//
// With kn = k / sqrt(|k|^2 + 1e-6) and qn likewise, the gated delta rule
//   S_t = e^{g_t} (I - beta_t kn_t kn_t^T) S_{t-1} + beta_t kn_t v_t^T,  o_t = S_t^T qn_t
// is the WKV7 recurrence S_t = diag(e^{w_t}) S_{t-1} + a_t (b_t^T S_{t-1}) + k_t v_t^T,
// o_t = S_t^T r_t, for the operands
//   r = qn,  w = g (every channel),  k = beta kn,  a = -e^{g} beta kn,  b = kn.
// The gradients therefore come in three launches on the caller's stream:
//  1. gdn_map_kernel writes those operands (and v, d_o) as fp32 rows into the
//     workspace, so the WKV7 backward sees them without rounding;
//  2. the WKV7 backward (fp32 I/O) turns d_o and d_final_state into the
//     gradients of r, w, k, v, a, b and of the initial state;
//  3. gdn_post_kernel applies the chain rule back to the Gated DeltaNet
//     inputs, per (token, head):
//        dkn   = beta dk - e^{g} beta da + db,     dqn = dr,
//        dq    = (dqn - qn (qn . dqn)) / sqrt(|q|^2 + 1e-6),  dk likewise,
//        dbeta = kn . dk_w - e^{g} kn . da,        dg = sum_c dw_c + a . da.
// A shared initial state ([1,H,K,V], B > 1) is expanded to one row per
// sequence before step 2, and its gradient is the sum over the sequences,
// taken in sequence order afterwards.
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace wkv7 {
namespace {

constexpr float kNormEps = 1e-6f;

template <typename T> struct g4;
template <> struct g4<float> {
    __device__ __forceinline__ static f32x4 load(const float *p, size_t i) { return *(const f32x4 *)(p + i); }
    __device__ __forceinline__ static void store(float *p, size_t i, f32x4 x) { *(f32x4 *)(p + i) = x; }
};
template <> struct g4<uint16_t> {
    __device__ __forceinline__ static f32x4 load(const uint16_t *p, size_t i)
    {
        const u32x2 u = *(const u32x2 *)(p + i);
        return f32x4{bf16_lo(u[0]), bf16_hi(u[0]), bf16_lo(u[1]), bf16_hi(u[1])};
    }
    __device__ __forceinline__ static void store(uint16_t *p, size_t i, f32x4 x)
    {
        *(u32x2 *)(p + i) = u32x2{cvt2_bits(x[0], x[1]), cvt2_bits(x[2], x[3])};
    }
};

// Sum over the D/4 lanes that share one (token, head) row; the groups are
// aligned blocks of D/4 lanes, so xor partners stay inside the group.
template <int D>
__device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int m = 1; m < D / 4; m <<= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

// Fp32 workspace rows of the mapped operands and of their gradients.
struct Planes {
    float *r, *w, *k, *v, *a, *b, *d_o;
    float *dr, *dw, *dk, *dv, *da, *db;
};

// One thread per four channels of one (token, head) row; rows are
// ((b T + t) H + h), the [B,T,H] index of g and beta.
template <int D, typename T_IO>
__global__ __launch_bounds__(256) void gdn_map_kernel(size_t nrows, const T_IO *__restrict__ q,
                                                      const T_IO *__restrict__ k, const T_IO *__restrict__ v,
                                                      const T_IO *__restrict__ g, const T_IO *__restrict__ beta,
                                                      const T_IO *__restrict__ d_o, Planes P)
{
    constexpr int GL = D / 4, RPB = 256 / GL;
    const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / GL;
    const bool valid = row < nrows;
    const size_t rr = valid ? row : nrows - 1;   // whole groups are valid or not: loads stay in bounds
    const size_t gi = rr * D + 4 * (threadIdx.x % GL);
    const f32x4 q4 = g4<T_IO>::load(q, gi), k4 = g4<T_IO>::load(k, gi);
    const float gg = io<T_IO>::load(g, rr), bt = io<T_IO>::load(beta, rr);
    const float iq = 1.0f / sqrtf(group_sum<D>(dot4(q4, q4)) + kNormEps);
    const float ik = 1.0f / sqrtf(group_sum<D>(dot4(k4, k4)) + kNormEps);
    if (!valid) return;
    const f32x4 kn = k4 * ik;
    g4<float>::store(P.r, gi, q4 * iq);
    g4<float>::store(P.w, gi, f32x4{gg, gg, gg, gg});
    g4<float>::store(P.k, gi, kn * bt);
    g4<float>::store(P.a, gi, kn * (-__expf(gg) * bt));
    g4<float>::store(P.b, gi, kn);
    g4<float>::store(P.v, gi, g4<T_IO>::load(v, gi));
    g4<float>::store(P.d_o, gi, g4<T_IO>::load(d_o, gi));
}

template <int D, typename T_IO>
__global__ __launch_bounds__(256) void gdn_post_kernel(size_t nrows, const T_IO *__restrict__ q,
                                                       const T_IO *__restrict__ k, const T_IO *__restrict__ g,
                                                       const T_IO *__restrict__ beta, Planes P,
                                                       T_IO *__restrict__ dq, T_IO *__restrict__ dk,
                                                       T_IO *__restrict__ dv, T_IO *__restrict__ dg,
                                                       T_IO *__restrict__ dbeta)
{
    constexpr int GL = D / 4, RPB = 256 / GL;
    const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / GL;
    const bool valid = row < nrows;
    const size_t rr = valid ? row : nrows - 1;
    const int c4 = 4 * (threadIdx.x % GL);
    const size_t gi = rr * D + c4;
    const f32x4 q4 = g4<T_IO>::load(q, gi), k4 = g4<T_IO>::load(k, gi);
    const float gg = io<T_IO>::load(g, rr), bt = io<T_IO>::load(beta, rr);
    const float iq = 1.0f / sqrtf(group_sum<D>(dot4(q4, q4)) + kNormEps);
    const float ik = 1.0f / sqrtf(group_sum<D>(dot4(k4, k4)) + kNormEps);
    const f32x4 qn = q4 * iq, kn = k4 * ik;
    const f32x4 gr = g4<float>::load(P.dr, gi), gw = g4<float>::load(P.dw, gi);
    const f32x4 gk = g4<float>::load(P.dk, gi), ga = g4<float>::load(P.da, gi);
    const f32x4 gb = g4<float>::load(P.db, gi);
    const float eg = __expf(gg);
    const f32x4 dkn = gk * bt - ga * (eg * bt) + gb;
    const float pq = group_sum<D>(dot4(qn, gr));
    const float pk = group_sum<D>(dot4(kn, dkn));
    const float kdk = group_sum<D>(dot4(kn, gk));
    const float kda = group_sum<D>(dot4(kn, ga));
    const float sw = group_sum<D>(gw[0] + gw[1] + gw[2] + gw[3]);
    if (!valid) return;
    g4<T_IO>::store(dq, gi, (gr - qn * pq) * iq);
    g4<T_IO>::store(dk, gi, (dkn - kn * pk) * ik);
    g4<T_IO>::store(dv, gi, g4<float>::load(P.dv, gi));
    if (c4 == 0) {
        io<T_IO>::store(dbeta, rr, kdk - eg * kda);
        io<T_IO>::store(dg, rr, sw - eg * bt * kda);   // a . da with a = -e^{g} beta kn
    }
}

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

template <int D, typename T_IO>
hipError_t launch_gdn_bwd_d(const GdnBwdArgs &p, hipStream_t stream)
{
    const size_t nrows = (size_t)p.B * p.T * p.H, plane = up(nrows * D * sizeof(float));
    const size_t per_state = (size_t)p.H * D * D, states = up((size_t)p.B * per_state * sizeof(float));
    char *ws = (char *)p.ws;
    float *pl[13];
    for (int i = 0; i < 13; ++i) pl[i] = (float *)(ws + i * plane);
    float *s0x = (float *)(ws + 13 * plane);
    float *ds0x = (float *)(ws + 13 * plane + states);
    void *wkv_ws = ws + 13 * plane + 2 * states;
    const Planes P{pl[0], pl[1], pl[2], pl[3], pl[4], pl[5], pl[6], pl[7], pl[8], pl[9], pl[10], pl[11], pl[12]};

    constexpr int RPB = 256 / (D / 4);
    const unsigned grid_rows = (unsigned)((nrows + RPB - 1) / RPB);
    const unsigned grid_state = (unsigned)((per_state / 4 + 255) / 256);
    const bool shared = p.s0 && p.n_state == 1 && p.B > 1;

    hipLaunchKernelGGL((gdn_map_kernel<D, T_IO>), dim3(grid_rows), dim3(256), 0, stream, nrows,
                       (const T_IO *)p.q, (const T_IO *)p.k, (const T_IO *)p.v, (const T_IO *)p.g,
                       (const T_IO *)p.beta, (const T_IO *)p.d_o, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float *s0 = p.s0;
    if (shared) {
        hipLaunchKernelGGL(expand_state_kernel, dim3(grid_state), dim3(256), 0, stream, p.s0, s0x, per_state, p.B);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        s0 = s0x;
    }
    float *d_s0 = p.d_s0 ? (shared ? ds0x : p.d_s0) : nullptr;
    const BwdArgs wa{p.B, p.T, p.H, D, P.r, P.w, P.k, P.v, P.a, P.b, s0, nullptr, P.d_o, p.d_sf,
                     P.dr, P.dw, P.dk, P.dv, P.da, P.db, d_s0, wkv_ws};
    if ((e = launch_backward(0, wa, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_post_kernel<D, T_IO>), dim3(grid_rows), dim3(256), 0, stream, nrows,
                       (const T_IO *)p.q, (const T_IO *)p.k, (const T_IO *)p.g, (const T_IO *)p.beta, P,
                       (T_IO *)p.dq, (T_IO *)p.dk, (T_IO *)p.dv, (T_IO *)p.dg, (T_IO *)p.dbeta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (shared && p.d_s0) {
        hipLaunchKernelGGL(sum_states_kernel, dim3(grid_state), dim3(256), 0, stream, ds0x, p.d_s0, per_state, p.B);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

size_t gdn_bwd_workspace_bytes(int B, int T, int H, int D)
{
    const size_t nrows = (size_t)B * T * H;
    return 13 * up(nrows * D * sizeof(float)) + 2 * up((size_t)B * H * D * D * sizeof(float)) +
           bwd_workspace_bytes(B, T, H, D);
}

hipError_t launch_gdn_backward(int dtype, const GdnBwdArgs &p, hipStream_t stream)
{
    if (p.D == 64) return dtype == 0 ? launch_gdn_bwd_d<64, float>(p, stream) : launch_gdn_bwd_d<64, uint16_t>(p, stream);
    return dtype == 0 ? launch_gdn_bwd_d<128, float>(p, stream) : launch_gdn_bwd_d<128, uint16_t>(p, stream);
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

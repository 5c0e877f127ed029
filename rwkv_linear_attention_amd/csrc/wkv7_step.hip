// Single-token WKV7 decode, state updated in place (rwkv-ops README, section
// "rwkv7_op_rnn 使用方法": the T = 1 case of the forward).
//
//   sb = b^T S ;  S = diag(exp(w)) S + a sb^T + k v^T ;  o = S^T r
//
// The state read and write dominate (2 x 4*D*D bytes per (b, h) against
// ~12*D bytes of inputs), so the kernel is an HBM stream.  One wave owns CW
// state columns of one (b, h): lane (cg, rg) holds rows [16*rg, 16*rg + 16)
// of columns [4*cg, 4*cg + 4) as 16 float4 registers, loaded with 16-byte
// accesses (each wave-wide load touches whole 128-byte lines).  b^T S and
// S^T r are in-lane FMA chains over 16 rows followed by a butterfly across
// the row groups.  D = 64: one wave covers the whole state (16 column groups
// x 4 row groups); D = 128: four waves, each 32 columns (8 x 8).
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace wkv7 {

template <typename T_IO> struct vec16;   // 16 consecutive elements
template <> struct vec16<uint16_t> {
    __device__ __forceinline__ static void load(const uint16_t *p, float *out) {
        const u32x4 *q = (const u32x4 *)p;
        u32x4 x0 = q[0], x1 = q[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_lo(x0[i]);  out[2 * i + 1] = bf16_hi(x0[i]);
            out[8 + 2 * i] = bf16_lo(x1[i]);  out[8 + 2 * i + 1] = bf16_hi(x1[i]);
        }
    }
};
template <> struct vec16<float> {
    __device__ __forceinline__ static void load(const float *p, float *out) {
        const f32x4 *q = (const f32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 x = q[i];
            out[4 * i] = x[0]; out[4 * i + 1] = x[1]; out[4 * i + 2] = x[2]; out[4 * i + 3] = x[3];
        }
    }
};

// GDN = true: Gated DeltaNet decode (rwkv-ops README, section
// "gdn_recurrent 使用方法", gated_delta_net_recurrent_single_step) in the same
// slots: r = q, k = k, v = v, w = gate g [B,H], a = strength beta [B,H] (b
// unused).  q and k are L2-normalised here (1e-6 added to the squared
// length), and the step is the generalized-delta-rule step with r = qn,
// w = g, k = beta kn, a = -e^g beta kn, b = kn.  The state is read from
// s_in (row bh, or row h of a single shared state when n_in == 1; nullptr
// reads zeros) and written to s_out (row bh); the two may be the same
// buffer when every sequence has its own row.
template <int D, typename T_IO, bool GDN>
__global__ __launch_bounds__(256) void step_kernel(
    int nwaves, int H, const T_IO *__restrict__ r, const T_IO *__restrict__ w,
    const T_IO *__restrict__ k, const T_IO *__restrict__ v, const T_IO *__restrict__ a,
    const T_IO *__restrict__ b, const float *s_in, int n_in, float *s_out, T_IO *__restrict__ o)
{
    constexpr int CW = (D == 64) ? 64 : 32;   // columns per wave
    constexpr int NCG = CW / 4;               // column groups per wave
    constexpr int WPS = D / CW;               // waves per (b, h)
    const int gw = blockIdx.x * 4 + threadIdx.x / kWave;
    if (gw >= nwaves) return;
    const int lane = threadIdx.x % kWave;
    const int bh = gw / WPS;
    const int cs = gw % WPS;
    const int cg = lane % NCG, rg = lane / NCG;
    const int col0 = cs * CW + cg * 4;
    const int row0 = rg * 16;

    const size_t off = (size_t)row0 * D + col0;
    const int sidx = (GDN && n_in == 1) ? bh % H : bh;
    float *Sp = s_out + (size_t)bh * D * D + off;
    f32x4 S[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        S[i] = s_in ? *(const f32x4 *)(s_in + (size_t)sidx * D * D + off + (size_t)i * D) : f32x4{0.f, 0.f, 0.f, 0.f};

    const size_t vb = (size_t)bh * D;
    float rv[16], ev[16], kv[16], av[16], bv[16];
    float vj[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vj[c] = io<T_IO>::load(v, vb + col0 + c);
    if constexpr (GDN) {
        float qv[16], kr[16];
        vec16<T_IO>::load(r + vb + row0, qv);
        vec16<T_IO>::load(k + vb + row0, kr);
        float nq = 0.f, nk = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            nq = fmaf(qv[i], qv[i], nq);
            nk = fmaf(kr[i], kr[i], nk);
        }
#pragma unroll
        for (int m = NCG; m < kWave; m <<= 1) {
            nq = xor_sum(nq, m);
            nk = xor_sum(nk, m);
        }
        const float iq = 1.0f / sqrtf(nq + 1e-6f), ik = 1.0f / sqrtf(nk + 1e-6f);
        const float gate = io<T_IO>::load(w, bh), beta = io<T_IO>::load(a, bh);
        const float eg = __expf(gate);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float kn = kr[i] * ik;
            rv[i] = qv[i] * iq;
            ev[i] = eg;
            kv[i] = beta * kn;
            av[i] = -eg * beta * kn;
            bv[i] = kn;
        }
    } else {
        vec16<T_IO>::load(r + vb + row0, rv);
        vec16<T_IO>::load(w + vb + row0, ev);
        vec16<T_IO>::load(k + vb + row0, kv);
        vec16<T_IO>::load(a + vb + row0, av);
        vec16<T_IO>::load(b + vb + row0, bv);
#pragma unroll
        for (int i = 0; i < 16; ++i) ev[i] = __expf(ev[i]);
    }

    float sb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            p0 = fmaf(bv[i], S[i][c], p0);
            p1 = fmaf(bv[i + 1], S[i + 1][c], p1);
        }
        sb[c] = p0 + p1;
    }
#pragma unroll
    for (int m = NCG; m < kWave; m <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) sb[c] = xor_sum(sb[c], m);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) S[i][c] = fmaf(ev[i], S[i][c], fmaf(av[i], sb[c], kv[i] * vj[c]));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) *(f32x4 *)(Sp + (size_t)i * D) = S[i];

    float ov[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            p0 = fmaf(rv[i], S[i][c], p0);
            p1 = fmaf(rv[i + 1], S[i + 1][c], p1);
        }
        ov[c] = p0 + p1;
    }
#pragma unroll
    for (int m = NCG; m < kWave; m <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) ov[c] = xor_sum(ov[c], m);
    }
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) io<T_IO>::store(o, vb + col0 + c, ov[c]);
    }
}

template <int D, typename T_IO>
static hipError_t launch_st(const StepArgs &p, hipStream_t stream)
{
    constexpr int WPS = (D == 64) ? 1 : 4;
    const long long nwaves = (long long)p.B * p.H * WPS;
    const dim3 grid((unsigned)((nwaves + 3) / 4)), block(256);
    if (p.gdn)
        hipLaunchKernelGGL((step_kernel<D, T_IO, true>), grid, block, 0, stream, (int)nwaves, p.H,
                           (const T_IO *)p.r, (const T_IO *)p.w, (const T_IO *)p.k, (const T_IO *)p.v,
                           (const T_IO *)p.a, (const T_IO *)p.b, p.state_in, p.n_state_in, p.state,
                           (T_IO *)p.o);
    else
        hipLaunchKernelGGL((step_kernel<D, T_IO, false>), grid, block, 0, stream, (int)nwaves, p.H,
                           (const T_IO *)p.r, (const T_IO *)p.w, (const T_IO *)p.k, (const T_IO *)p.v,
                           (const T_IO *)p.a, (const T_IO *)p.b, p.state, p.B, p.state, (T_IO *)p.o);
    return hipGetLastError();
}

hipError_t launch_step(int dtype, const StepArgs &p, hipStream_t stream)
{
    if (p.D == 64) return dtype == 0 ? launch_st<64, float>(p, stream) : launch_st<64, uint16_t>(p, stream);
    return dtype == 0 ? launch_st<128, float>(p, stream) : launch_st<128, uint16_t>(p, stream);
}

}  // namespace wkv7

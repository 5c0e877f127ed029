// Token-by-token WKV7 forward in fp32 (fp32 or bf16 I/O).
//
// Recurrence (rwkv-ops README, section "rwkv7op 使用方法"; update read as the
// generalized delta rule): for every (b, h) and token t with mask != 0
//   sb = b_t^T S ;  S = diag(exp(w_t)) S + a_t sb^T + k_t v_t^T
// and for every token  o_t = S^T r_t.
//
// Sequences come either as [B,T,H,D] arrays or packed ([T_total,H,D] with
// cu_seqlens offsets and a state_map into a pool of initial states).
//
// One workgroup per (b, h) with D/16 waves; wave w owns state columns
// [16w, 16w+16).  Lane (j = l%16, g = l/16) keeps rows [g*D/4, (g+1)*D/4) of
// column 16w + j in VGPRs, so b^T S and S^T r are in-lane FMA chains over D/4
// rows plus a 4-way cross-lane sum.  Tokens are staged in LDS 16 at a time
// (fp32, exp(w) precomputed); all lanes of a row group read the same LDS
// address (broadcast).  The next block's inputs are loaded into registers
// (one thread per token and four channels) while the current block runs.
// This path is latency-bound and serves fp32 I/O, short sequences and few
// (b, h) pairs.
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace wkv7 {

// GDN = true takes Gated DeltaNet inputs in the same slots: r = q, k = k,
// v = v, w = gate g [.., H], a = strength beta [.., H] (b and mask unused);
// each staged token is turned into the generalized-delta-rule operands
// r = qn, w = g, k = beta kn, a = -e^g beta kn, b = kn (q, k L2-normalised;
// rwkv-ops README, section "gdn_recurrent 使用方法", read as the gated delta
// rule).
template <int D, typename T_IO, bool GDN>
__global__ __launch_bounds__(D * 4) void recurrent_kernel(
    int T, int H, const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ state_map,
    int n_state, const T_IO *__restrict__ r, const T_IO *__restrict__ w,
    const T_IO *__restrict__ k, const T_IO *__restrict__ v, const T_IO *__restrict__ a,
    const T_IO *__restrict__ b, const float *__restrict__ s0, const uint8_t *__restrict__ mask,
    T_IO *__restrict__ o, float *__restrict__ sf)
{
    constexpr int TB = 16;          // tokens staged per block
    constexpr int RPL = D / 4;      // state rows per lane
    constexpr int NT = D * 4;       // threads
    __shared__ float s_ew[TB][D], s_a[TB][D], s_b[TB][D], s_k[TB][D], s_r[TB][D], s_v[TB][D];

    const int bh = blockIdx.x;
    // Sequence sq: tokens [tok0, tok0 + Tn) of the token axis (packed form:
    // from cu_seqlens, clamped into range), initial state row sidx of the
    // state pool (-1: zeros).
    const int sq = bh / H, h = bh % H;
    size_t tok0;
    int Tn, sidx = sq;
    if (cu_seqlens) {
        const int t_beg = min(max(cu_seqlens[sq], 0), T);
        const int t_end = min(max(cu_seqlens[sq + 1], t_beg), T);
        tok0 = (size_t)t_beg;
        Tn = t_end - t_beg;
    } else {
        tok0 = (size_t)sq * T;
        Tn = T;
    }
    if (state_map) {
        sidx = state_map[sq];
        if (sidx < 0 || sidx >= n_state) sidx = -1;
    } else if (n_state == 1) {
        sidx = 0;   // one initial state shared by every sequence
    }
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int col = wave * 16 + (lane & 15);
    const int g = lane >> 4;
    const int row0 = g * RPL;

    float S[RPL];
    const size_t st_base = (size_t)bh * D * D;
    const size_t st_in = ((size_t)(sidx < 0 ? 0 : sidx) * H + h) * D * D;
#pragma unroll
    for (int i = 0; i < RPL; ++i) S[i] = 0.0f;
    if (s0 && sidx >= 0) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) S[i] = s0[st_in + (size_t)(row0 + i) * D + col];
    }

    // Inputs of one staged block: thread (tp, cp) holds channels cp .. cp + 3
    // of token tp (zeros past the sequence's end); the D/4 threads of a token
    // are adjacent lanes.  Generalized rule: w, a, b, k, r, v.  Gated
    // DeltaNet: q, k, v in slots 4, 3, 5 and the token's gate and strength.
    static_assert(NT == TB * D / 4, "one thread per (token, 4 channels)");
    const int tp = tid / (D / 4), cp = 4 * (tid % (D / 4));
    using R4 = raw4<T_IO>;
    typename R4::type pf[6];
    int pup = 0;
    float pg = 0.f, pb = 0.f;
    auto fetch = [&](int t0) {
        const bool valid = t0 + tp < Tn;
        const size_t gi = ((tok0 + t0 + tp) * H + h) * D + cp;
        if constexpr (GDN) {
            pf[4] = valid ? R4::load(r, gi) : R4::zero();
            pf[3] = valid ? R4::load(k, gi) : R4::zero();
            pf[5] = valid ? R4::load(v, gi) : R4::zero();
            const size_t si = (tok0 + t0 + tp) * H + h;
            pg = valid ? io<T_IO>::load(w, si) : 0.f;
            pb = valid ? io<T_IO>::load(a, si) : 0.f;
        } else {
            const T_IO *src[6] = {w, a, b, k, r, v};
#pragma unroll
            for (int x = 0; x < 6; ++x) pf[x] = valid ? R4::load(src[x], gi) : R4::zero();
            pup = valid && (mask ? mask[tok0 + t0 + tp] != 0 : 1);
        }
    };
    if (Tn > 0) fetch(0);

    for (int t0 = 0; t0 < Tn; t0 += TB) {
        const int nt = min(TB, Tn - t0);
        __syncthreads();
        if constexpr (GDN) {
            // qn = q / |q|, kn = k / |k| (norms over the token's lanes), then
            // r = qn, w = g, k = beta kn, a = -e^g beta kn, b = kn
            const f32x4 q4 = R4::f32(pf[4]), k4 = R4::f32(pf[3]);
            const float iq = inv_norm<D>(q4), ik = inv_norm<D>(k4);
            const f32x4 kn = k4 * ik;
            const float eg = __expf(pg);
            *(f32x4 *)&s_r[tp][cp] = q4 * iq;
            *(f32x4 *)&s_b[tp][cp] = kn;
            *(f32x4 *)&s_k[tp][cp] = kn * pb;
            *(f32x4 *)&s_a[tp][cp] = kn * (-eg * pb);
            *(f32x4 *)&s_ew[tp][cp] = f32x4{eg, eg, eg, eg};
            *(f32x4 *)&s_v[tp][cp] = R4::f32(pf[5]);
            if (t0 + TB < Tn) fetch(t0 + TB);
        } else {
            // A token that does not update becomes an exact identity step
            // (e^w = 1, a = b = k = v = 0), whatever its inputs hold, even
            // inf or nan; its r still produces an output.
            const f32x4 wv = R4::f32(pf[0]), z4 = {0.f, 0.f, 0.f, 0.f};
            f32x4 ew;
#pragma unroll
            for (int i = 0; i < 4; ++i) ew[i] = pup ? __expf(wv[i]) : 1.0f;
            *(f32x4 *)&s_ew[tp][cp] = ew;
            *(f32x4 *)&s_a[tp][cp] = pup ? R4::f32(pf[1]) : z4;
            *(f32x4 *)&s_b[tp][cp] = pup ? R4::f32(pf[2]) : z4;
            *(f32x4 *)&s_k[tp][cp] = pup ? R4::f32(pf[3]) : z4;
            *(f32x4 *)&s_r[tp][cp] = R4::f32(pf[4]);
            *(f32x4 *)&s_v[tp][cp] = pup ? R4::f32(pf[5]) : z4;
            if (t0 + TB < Tn) fetch(t0 + TB);
        }
        __syncthreads();

        // Every staged token updates (a masked one as the identity), so the
        // steps have no branch and a full block is unrolled: the loads of a
        // token's operands can then run ahead of the previous token's chain.
        auto token = [&](int tl) {
            {
                float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
                for (int i = 0; i < RPL; i += 4) {
                    p0 += s_b[tl][row0 + i + 0] * S[i + 0];
                    p1 += s_b[tl][row0 + i + 1] * S[i + 1];
                    p2 += s_b[tl][row0 + i + 2] * S[i + 2];
                    p3 += s_b[tl][row0 + i + 3] * S[i + 3];
                }
                float sb = (p0 + p1) + (p2 + p3);
                sb = xsum16(sb);
                sb = xsum32(sb);
                const float vj = s_v[tl][col];
#pragma unroll
                for (int i = 0; i < RPL; ++i)
                    S[i] = fmaf(s_ew[tl][row0 + i], S[i], fmaf(s_a[tl][row0 + i], sb, s_k[tl][row0 + i] * vj));
            }
            float q0 = 0.f, q1 = 0.f, q2 = 0.f, q3 = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; i += 4) {
                q0 += s_r[tl][row0 + i + 0] * S[i + 0];
                q1 += s_r[tl][row0 + i + 1] * S[i + 1];
                q2 += s_r[tl][row0 + i + 2] * S[i + 2];
                q3 += s_r[tl][row0 + i + 3] * S[i + 3];
            }
            float ov = (q0 + q1) + (q2 + q3);
            ov = xsum16(ov);
            ov = xsum32(ov);
            if (g == 0) io<T_IO>::store(o, ((tok0 + t0 + tl) * H + h) * D + col, ov);
        };
        if (nt == TB) {
#pragma unroll
            for (int tl = 0; tl < TB; ++tl) token(tl);
        } else {
            for (int tl = 0; tl < nt; ++tl) token(tl);
        }
    }
    if (sf) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) sf[st_base + (size_t)(row0 + i) * D + col] = S[i];
    }
}

template <int D, typename T_IO>
static hipError_t launch_rec(const FwdArgs &p, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.B * p.H)), block(D * 4);
    if (p.gdn) {
        hipLaunchKernelGGL((recurrent_kernel<D, T_IO, true>), grid, block, 0, stream, p.T, p.H, p.cu_seqlens,
                           p.state_map, p.n_state,
                           (const T_IO *)p.r, (const T_IO *)p.w, (const T_IO *)p.k, (const T_IO *)p.v,
                           (const T_IO *)p.a, (const T_IO *)p.b, p.s0, p.mask, (T_IO *)p.o, p.sf);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((recurrent_kernel<D, T_IO, false>), grid, block, 0, stream, p.T, p.H, p.cu_seqlens,
                       p.state_map, p.n_state,
                       (const T_IO *)p.r, (const T_IO *)p.w, (const T_IO *)p.k, (const T_IO *)p.v,
                       (const T_IO *)p.a, (const T_IO *)p.b, p.s0, p.mask, (T_IO *)p.o, p.sf);
    return hipGetLastError();
}

hipError_t launch_recurrent(int dtype, const FwdArgs &p, hipStream_t stream)
{
    if (p.D == 64) return dtype == 0 ? launch_rec<64, float>(p, stream) : launch_rec<64, uint16_t>(p, stream);
    return dtype == 0 ? launch_rec<128, float>(p, stream) : launch_rec<128, uint16_t>(p, stream);
}

}  // namespace wkv7

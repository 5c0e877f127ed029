// Chunked WKV7 forward for fp32 I/O, on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32), K = V = 64 or 128.
//
// The recurrence (rwkv-ops README, section "rwkv7op 使用方法", read as the
// generalized delta rule) is evaluated 16 tokens at a time in the same chunk
// form as the bf16 kernel (wkv7_chunked.hip):
//
//   X  = B~ S + M_bk V,    U = T X,    T = (I - M_ba)^-1
//   O  = R~ S + M_ra U + M_rk V
//   S' = diag(e^{G_L}) (S + A^^T U + K^^T V)
//
// with G the per-channel inclusive decay prefix inside the chunk, R~ = r e^G,
// B~ = b e^{G_{t-1}}, A^ = a e^{-G}, K^ = k e^{-G}, M_ba = B~ A^^T and
// M_bk = B~ K^^T strictly lower, M_ra = R~ A^^T and M_rk = R~ K^^T lower with
// the diagonal.  Every product runs on fp32 operands with fp32 accumulation:
// splitting fp32 operands into bf16 pieces (three bf16 products per fp32
// product) measured, in a numpy emulation of this chunk form, up to 7e-5
// absolute error on the outputs against the fp64 recurrence -- too close to
// the 1e-4 bound of fp32 I/O -- while fp32 products gave 2.4e-6.
//
// Work layout: one workgroup per (sequence, head), D/16 waves; wave i keeps
// state columns 16 i .. 16 i + 15 in MFMA accumulator registers (lane
// (m, q) holds rows 16 ti + 4 q + r of column 16 i + m) for the whole
// sequence.  Per chunk all waves stage the chunk's inputs into LDS (each
// thread four channels of one token, a channel group's 16 tokens in one
// 16-lane row; at D = 64 the next chunk's loads are in flight meanwhile), each thread
// forms its decay prefix by a scan across its row, the four waves 0..3 form
// one chunk matrix each, T is formed (D = 64: by every wave, forward
// substitution with one column per lane; D = 128: by wave 0 on the matrix
// cores, nilpotent doubling) and then each wave runs the products of its own
// columns.  Contractions over state rows or chunk tokens take the
// index in the order the accumulator layout holds it, so the state and the
// intermediate tiles feed the matrix cores straight from registers; the
// output is formed transposed (O^T = S^T R~^T + U^T M_ra^T + V^T M_rk^T) so
// that each lane stores four adjacent outputs of one token.  A chunk with a
// positive w, or whose decay reaches e^-60, runs token by token instead (the
// split factors e^{-G} would leave the fp32 range).  A token with mask 0, or
// past the sequence end, gets w = a = k = b = v = 0: an exact identity step.
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace wkv7 {
namespace {

constexpr int kL = 16;
constexpr float kMinChunkLogDecay = -60.0f;

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D> struct F32Cfg {
    static_assert(D == 64 || D == 128, "head size");
    static constexpr int NW = D / 16;           // waves, one 16-column state slice each
    static constexpr int NTH = 64 * NW;         // threads: four channels of one token each
    static constexpr int NTILE = D / 16;        // 16-row tiles of the state
    static constexpr int LD = D + 4;            // padded row, floats
};

// One chunk's tiles.  Tokens are rows; R, B, A, K hold the scaled operands
// (raw r, b, a, k on the token-by-token path).
template <int D> struct alignas(16) F32Buf {
    static constexpr int LD = F32Cfg<D>::LD;
    float W[kL][LD];          // w (0 where the token does not update)
    float V[kL][LD];          // v (likewise)
    float R[kL][LD], B[kL][LD], A[kL][LD], K[kL][LD];
    float M[4][kL][kL + 4];   // M_ba, M_bk, M_ra, M_rk
    float EGL[D];             // e^{G_L}
    int upd[kL];
};

// One chunk buffer, with a barrier at the end of each chunk before the next
// one is staged.  At D = 64 that is 36.9 KB of LDS, room for three
// workgroups per CU (their VGPRs fit too).  Two buffers (68.5 KB, no
// end-of-chunk barrier, two workgroups per CU) measured 1.327 ms against
// 1.283 ms at B8 T4096 H64 (512 workgroups), with bit-identical results; a
// 128-VGPR cap for four workgroups per CU spilled and took 1.66 ms.
template <int D> struct alignas(16) F32Lds {
    F32Buf<D> buf;
    // D = 64: each wave's copy of T.  D = 128: T^T as wave 0's accumulator,
    // lane (q, m) at [0][m][4q].
    float T[D == 64 ? F32Cfg<D>::NW : 1][kL][kL + 4];
};

template <int D, bool ORDERED>
__global__ __launch_bounds__(F32Cfg<D>::NTH) __attribute__((amdgpu_waves_per_eu(D == 128 ? 4 : 3))) void
chunked_f32_kernel(
    int T, int H, const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ state_map, int n_state,
    const float *__restrict__ r, const float *__restrict__ w, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ a, const float *__restrict__ b,
    const float *__restrict__ s0, const uint8_t *__restrict__ mask, float *__restrict__ o,
    float *__restrict__ sf)
{
    using C = F32Cfg<D>;
    constexpr int NTILE = C::NTILE;
    __shared__ __attribute__((aligned(16))) F32Lds<D> s;
    const int bh = blockIdx.x;
    const int h = bh % H;
    // Packed batches of few sequences run longest first: workgroup bh takes
    // the sequence of rank bh / H by length (ORDERED, chosen on the host:
    // use_longest_first).
    int sq = bh / H, lf_tb = 0, lf_tn = 0;
    if constexpr (ORDERED) {
        __shared__ int lf_beg[kLongestFirstMax], lf_len[kLongestFirstMax], lf_rank[kLongestFirstMax], lf_pick[1];
        longest_first<1>(cu_seqlens, T, (int)gridDim.x / H, bh, H, lf_beg, lf_len, lf_rank, lf_pick);
        sq = lf_pick[0];
        lf_tb = lf_beg[sq];
        lf_tn = lf_len[sq];
    }
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int q = lane >> 4, m = lane & 15, c0 = 16 * wave;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};

    // Sequence sq: tokens [tok0, tok0 + Tn) of the (packed) token axis, and
    // initial-state row sidx of the pool (-1: zeros), clamped into range.
    size_t tok0;
    int Tn, sidx = sq;
    if (ORDERED) {
        tok0 = (size_t)lf_tb;   // clamped by longest_first
        Tn = lf_tn;
    } else if (cu_seqlens) {
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
    const int nck = (Tn + kL - 1) / kL;

    f32x4 St[NTILE];
    {
        const float *init = (s0 && sidx >= 0) ? s0 + ((size_t)sidx * H + h) * D * D : nullptr;
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
            for (int i = 0; i < 4; ++i) St[ti][i] = init ? init[(size_t)(16 * ti + 4 * q + i) * D + c0 + m] : 0.0f;
    }

    // Staging: thread (token tp, channels cp .. cp + 3), the 16 tokens of a
    // channel group in the 16 lanes of one row of a wave, so that the decay
    // prefix is a scan across the row.  D = 64: the next chunk's inputs are
    // loaded into registers while the current chunk runs.  D = 128: each
    // chunk's inputs are loaded at its start, which frees the registers for
    // a 128-VGPR limit: two workgroups then share a CU and cover each other's
    // latency (3.73 -> 3.65 ms at B16 T4096 H32; the limit spills a few
    // loop-invariant values).
    const int tp = lane & 15, cp = 4 * (4 * wave + (lane >> 4));
    // Every valid token's inputs are loaded; the mask byte is applied when
    // the chunk is staged (selects, so that nothing a masked token holds --
    // not even inf or nan -- reaches the state).
    f32x4 pr, pw, pk, pv, pa, pb;
    int pm = 1, pvalid = 0;
    auto fetch = [&](int c) {
        const int t = c * kL + tp;
        pvalid = t < Tn;
        const size_t gi = ((tok0 + (pvalid ? t : 0)) * H + h) * D + cp;
        pr = *(const f32x4 *)(r + gi);
        pw = *(const f32x4 *)(w + gi);
        pk = *(const f32x4 *)(k + gi);
        pv = *(const f32x4 *)(v + gi);
        pa = *(const f32x4 *)(a + gi);
        pb = *(const f32x4 *)(b + gi);
        if (mask) pm = mask[tok0 + (pvalid ? t : 0)];
    };
    if (D == 64 && nck > 0) fetch(0);

    for (int c = 0; c < nck; ++c) {
        F32Buf<D> &bf = s.buf;
        const int Lc = min(kL, Tn - c * kL);
        if (D == 128) fetch(c);
        // A token that does not update is an identity step whatever its
        // inputs hold: w = a = k = b = v = 0 (and r = 0 past the end).
        const bool up = pvalid && pm != 0;
        const f32x4 r4 = pvalid ? pr : z, w4 = up ? pw : z, k4 = up ? pk : z, a4 = up ? pa : z,
                    b4 = up ? pb : z, v4 = up ? pv : z;
        *(f32x4 *)&bf.W[tp][cp] = w4;
        *(f32x4 *)&bf.V[tp][cp] = v4;
        if (cp == 0) bf.upd[tp] = up;
        if (D == 64 && c + 1 < nck) fetch(c + 1);

        // Decay prefix of this thread's four channels, a scan over the row's
        // 16 lanes (tokens): G (token tp), the exclusive prefix Gp, and the
        // chunk total G_L.
        f32x4 G, Gp, GL;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            G[i] = row_scan16(w4[i]);
            Gp[i] = row_shr<1>(G[i], 0.0f);
            GL[i] = row_bcast15(G[i]);
        }
        int extreme = (w4[0] > 0.0f) | (w4[1] > 0.0f) | (w4[2] > 0.0f) | (w4[3] > 0.0f);
        extreme |= (GL[0] < kMinChunkLogDecay) | (GL[1] < kMinChunkLogDecay) | (GL[2] < kMinChunkLogDecay) |
                   (GL[3] < kMinChunkLogDecay);
        f32x4 eG, enG, eGp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            eG[i] = __expf(G[i]);
            enG[i] = __expf(-G[i]);
            eGp[i] = __expf(Gp[i]);
        }
        *(f32x4 *)&bf.R[tp][cp] = r4 * eG;
        *(f32x4 *)&bf.B[tp][cp] = b4 * eGp;
        *(f32x4 *)&bf.A[tp][cp] = a4 * enG;
        *(f32x4 *)&bf.K[tp][cp] = k4 * enG;
        if (tp == 0) {
            f32x4 egl;
#pragma unroll
            for (int i = 0; i < 4; ++i) egl[i] = __expf(GL[i]);
            *(f32x4 *)&bf.EGL[cp] = egl;
        }
        if (__syncthreads_or(extreme)) {
            // ---- exact path: token by token on the raw operands ----
            *(f32x4 *)&bf.R[tp][cp] = r4;
            *(f32x4 *)&bf.B[tp][cp] = b4;
            *(f32x4 *)&bf.A[tp][cp] = a4;
            *(f32x4 *)&bf.K[tp][cp] = k4;
            __syncthreads();
            for (int t = 0; t < Lc; ++t) {
                if (bf.upd[t]) {
                    float sb = 0.0f;
#pragma unroll
                    for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sb = fmaf(bf.B[t][16 * ti + 4 * q + i], St[ti][i], sb);
                    sb = xsum32(xsum16(sb));
                    const float vj = bf.V[t][c0 + m];
#pragma unroll
                    for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int row = 16 * ti + 4 * q + i;
                            St[ti][i] = fmaf(__expf(bf.W[t][row]), St[ti][i],
                                             fmaf(bf.A[t][row], sb, bf.K[t][row] * vj));
                        }
                }
                float ov = 0.0f;
#pragma unroll
                for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov = fmaf(bf.R[t][16 * ti + 4 * q + i], St[ti][i], ov);
                ov = xsum32(xsum16(ov));
                if (q == 0) o[((tok0 + c * kL + t) * H + h) * D + c0 + m] = ov;
            }
            __syncthreads();   // every wave is done with the buffer
            continue;
        }

        // ---- chunk matrices: wave i < 4 forms one (M_ba, M_bk, M_ra, M_rk) ----
        if (wave < 4) {
            const float(*P)[C::LD] = wave < 2 ? bf.B : bf.R;
            const float(*Q)[C::LD] = (wave & 1) ? bf.K : bf.A;
            f32x4 acc = z;
#pragma unroll
            for (int j0 = 0; j0 < D; j0 += 16) {
                const f32x4 x = *(const f32x4 *)&P[m][j0 + 4 * q];
                const f32x4 y = *(const f32x4 *)&Q[m][j0 + 4 * q];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = mfma_f32(x[i], y[i], acc);
            }
            const bool strict = wave < 2;   // M_ba, M_bk strictly lower; M_ra, M_rk with the diagonal
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * q + i;
                acc[i] = (strict ? row > m : row >= m) ? acc[i] : 0.0f;
                bf.M[wave][row][m] = acc[i];
            }
            if (D == 128 && wave == 0) {
                // T = (I - M_ba)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8), N = M_ba
                // strictly lower (N^16 = 0), on the matrix cores while waves 1..3
                // form the other chunk matrices: with the contraction index
                // permuted as in the products below, acc(X Y) = sum_st
                // mfma(acc(X^T)[st], acc(Y)[st]).  acc(T^T) goes to LDS; lane
                // (q, m) holds T[m][4q + i], the row operand of U = T X.
                auto mm = [](f32x4 aT, f32x4 b) {
                    f32x4 r4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < 4; ++st) r4 = mfma_f32(aT[st], b[st], r4);
                    return r4;
                };
                lds_wait();   // this wave's M_ba writes are complete before its transposed read
                const f32x4 nA = acc, nT = *(const f32x4 *)&bf.M[0][m][4 * q];   // acc(N), acc(N^T)
                f32x4 eye;
#pragma unroll
                for (int i = 0; i < 4; ++i) eye[i] = 4 * q + i == m ? 1.0f : 0.0f;
                const f32x4 n2 = mm(nT, nA), n2T = mm(nA, nT);
                const f32x4 n4 = mm(n2T, n2), n4T = mm(n2, n2T);
                const f32x4 n8 = mm(n4T, n4);
                const f32x4 p1T = mm(eye + n2, eye + nT);   // ((I + N)(I + N^2))^T
                const f32x4 p2T = mm(eye + n4, p1T);        // (P1 (I + N^4))^T
                *(f32x4 *)&s.T[0][m][4 * q] = mm(eye + n8, p2T);   // (I + N^8)^T P2^T = T^T
            }
        }
        __syncthreads();

        // ---- this wave's columns c0 .. c0 + 15 ----
        const float vm[4] = {bf.V[4 * q][c0 + m], bf.V[4 * q + 1][c0 + m], bf.V[4 * q + 2][c0 + m],
                             bf.V[4 * q + 3][c0 + m]};   // V[4q + i][c0 + m]
        // X = B~ S + M_bk V
        f32x4 X = z;
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti) {
            const f32x4 bt = *(const f32x4 *)&bf.B[m][16 * ti + 4 * q];
#pragma unroll
            for (int i = 0; i < 4; ++i) X = mfma_f32(bt[i], St[ti][i], X);
        }
        {
            const f32x4 mb = *(const f32x4 *)&bf.M[1][m][4 * q];
#pragma unroll
            for (int i = 0; i < 4; ++i) X = mfma_f32(mb[i], vm[i], X);
        }
        // O^T, state part (chunk-start state): S^T R~^T
        f32x4 Ot = z;
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti) {
            const f32x4 rt = *(const f32x4 *)&bf.R[m][16 * ti + 4 * q];
#pragma unroll
            for (int i = 0; i < 4; ++i) Ot = mfma_f32(St[ti][i], rt[i], Ot);
        }
        // ---- T = (I - M_ba)^-1, after the products above, which do not need
        // it, so that their matrix-core work overlaps the substitution (1.35
        // -> 1.33 ms at B8 T4096 H64).  D = 128: formed by wave 0 above
        // (eight waves would each repeat a substitution: 4.05 -> 3.89 ms
        // measured at B16 T4096 H32).  D = 64: this wave's copy, lane j < 16
        // solving column j; with four waves the substitution in every wave
        // measured faster than wave 0 alone on the matrix cores (1.35 against
        // 1.40 ms at B8 T4096 H64).  Column j = lane & 15 in every lane group:
        // row i of M_ba is read as four-float pieces (the same address in
        // every lane), all before the substitution, and each row's dot
        // product is split over two accumulators so that only its last term
        // waits for x_{i-1}. ----
        float(*Tw)[kL + 4] = s.T[D == 64 ? wave : 0];
        if constexpr (D == 64) {
            const int j = lane & 15;
            f32x4 mrow[kL - 1][4];
#pragma unroll
            for (int i = 1; i < kL; ++i)
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    if (4 * p < i) mrow[i - 1][p] = *(const f32x4 *)&bf.M[0][i][4 * p];
            float x[kL];
#pragma unroll
            for (int i = 0; i < kL; ++i) {
                float acc0 = i == j ? 1.0f : 0.0f, acc1 = 0.0f;
#pragma unroll
                for (int l = 0; l < i; ++l) {
                    const float mv = mrow[i - 1][l >> 2][l & 3];
                    if (l & 1) acc1 = fmaf(mv, x[l], acc1);
                    else acc0 = fmaf(mv, x[l], acc0);
                }
                x[i] = acc0 + acc1;
            }
            if (lane < kL) {
#pragma unroll
                for (int i = 0; i < kL; ++i) Tw[i][j] = x[i];
            }
            lds_wait();   // the wave's own T writes are complete before its reads
        }

        // U = T X
        f32x4 U = z;
        {
            // T[m][4q + i]: the wave's own copy (D = 64) or wave 0's T^T accumulator
            const f32x4 tr = *(const f32x4 *)&Tw[m][4 * q];
#pragma unroll
            for (int i = 0; i < 4; ++i) U = mfma_f32(tr[i], X[i], U);
        }
        // O^T += V^T M_rk^T + U^T M_ra^T
        {
            const f32x4 mk = *(const f32x4 *)&bf.M[3][m][4 * q];
            const f32x4 ma = *(const f32x4 *)&bf.M[2][m][4 * q];
#pragma unroll
            for (int i = 0; i < 4; ++i) Ot = mfma_f32(vm[i], mk[i], Ot);
#pragma unroll
            for (int i = 0; i < 4; ++i) Ot = mfma_f32(U[i], ma[i], Ot);
        }
        // S <- diag(e^{G_L}) (S + A^^T U + K^^T V)
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti) {
            f32x4 acc = St[ti];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = mfma_f32(bf.K[4 * q + i][16 * ti + m], vm[i], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = mfma_f32(bf.A[4 * q + i][16 * ti + m], U[i], acc);
            St[ti] = acc * *(const f32x4 *)&bf.EGL[16 * ti + 4 * q];
        }
        // O^T lane (m, q): token m, columns c0 + 4q .. + 3
        if (m < Lc) *(f32x4 *)(o + ((tok0 + c * kL + m) * H + h) * D + c0 + 4 * q) = Ot;
        __syncthreads();   // every wave is done with the buffer before the next chunk is staged
    }

    if (sf) {
        float *dst = sf + (size_t)(ORDERED ? sq * H + h : bh) * D * D;
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(size_t)(16 * ti + 4 * q + i) * D + c0 + m] = St[ti][i];
    }
}

template <int D>
hipError_t launch_f32(const FwdArgs &p, hipStream_t stream)
{
    const unsigned nbh = (unsigned)p.B * (unsigned)p.H;
    // packed calls of few sequences take them longest first
    auto kern = use_longest_first(p.cu_seqlens != nullptr, p.B, p.T) ? chunked_f32_kernel<D, true> : chunked_f32_kernel<D, false>;
    hipLaunchKernelGGL(kern, dim3(nbh), dim3(F32Cfg<D>::NTH), 0, stream, p.T, p.H, p.cu_seqlens,
                       p.state_map, p.n_state, (const float *)p.r, (const float *)p.w, (const float *)p.k,
                       (const float *)p.v, (const float *)p.a, (const float *)p.b, p.s0, p.mask, (float *)p.o,
                       p.sf);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunked_f32(const FwdArgs &p, hipStream_t stream)
{
    return p.D == 64 ? launch_f32<64>(p, stream) : launch_f32<128>(p, stream);
}

}  // namespace wkv7

// Backward of the WKV7 forward: gradients of r, w, k, v, a, b and of the
// initial state for upstream gradients d_o (of every output) and d_sf (of
// the final state).
//
// The recurrence (rwkv-ops README, section "rwkv7op 使用方法", which lists
// generalized_delta_rule as the trainable entry; update read as the
// generalized delta rule) is, per (b, h) and updating token t,
//   S_t = diag(e^{w_t}) S_{t-1} + a_t (b_t^T S_{t-1}) + k_t v_t^T,  o_t = S_t^T r_t.
// Its reverse-mode derivative carries dS = dL/dS_t backwards:
//   dS += r_t d_o_t^T;   dS_{t-1} = diag(e^{w_t}) dS + b_t (a_t^T dS).
//
// Two launches, with a caller-provided workspace and no allocation:
//  1. chain_kernel runs, side by side, (a) the forward recurrence in chunk
//     form, storing the state before every 16-token chunk (checkpoints), and (b) the dS recurrence backwards in chunk form,
//     storing for every chunk the gradient of the state at the chunk's end
//     with respect to everything after the chunk;
//  2. chunk_grad_kernel (one workgroup per (b, h, chunk), all chunks in
//     parallel) recomputes the chunk in its unrolled form from the chunk's
//     checkpoint and turns that end gradient into the token gradients.
//
// Chunk form (G the per-channel inclusive decay prefix inside the chunk,
// G_{t-1} the exclusive one; R~ = r e^G, B~ = b e^{G_{t-1}}, A^ = a e^{-G},
// K^ = k e^{-G}; M_xy the L x L products X Y^T, strictly lower for M_ba and
// M_bk, lower with the diagonal for M_ra and M_rk; T = (I - M_ba)^{-1}):
//   X = B~ S + M_bk V,  U = T X,  O = R~ S + M_ra U + M_rk V,
//   S' = diag(e^{G_L}) (S + A^T U + K^T V).
// Given dS' (the chunk-end gradient) and dO:
//   dY = diag(e^{G_L}) dS',  dU = A^ dY + M_ra^T dO,  dX = T^T dU,
//   dV = K^ dY + M_rk^T dO + M_bk^T dX,
//   dM_ra = dO U^T, dM_rk = dO V^T, dM_ba = dX U^T, dM_bk = dX V^T (masked),
//   dR~ = dO S^T + dM_ra A^ + dM_rk K^,   dB~ = dX S^T + dM_ba A^ + dM_bk K^,
//   dA^ = U dY^T + dM_ra^T R~ + dM_ba^T B~, dK^ = V dY^T + dM_rk^T R~ + dM_bk^T B~,
//   dr = dR~ e^G, db = dB~ e^{G_{t-1}}, da = dA^ e^{-G}, dk = dK^ e^{-G},
//   dw_m = sum_{t >= m} (dr_t r_t - da_t a_t - dk_t k_t + db_{t+1} b_{t+1})
//          + sum_j dS'[.,j] S'[.,j]     (the last term from the chunk end,
//          formed from S, U, V and dS' without reading the next checkpoint).
// A chunk whose decay reaches e^{-60} on some channel, or with a positive w,
// takes an exact token-by-token path instead (the split factors e^{-G} would
// leave the fp32 range).  All arithmetic is fp32: the products run on the
// fp32 matrix cores (v_mfma_f32_16x16x4_f32) over LDS tiles.
//
// Both launches also have a Gated DeltaNet mode (template flag GDN), used by
// wkv7_gdn_bwd: they form the generalized-rule operands of the gated delta
// rule from q, k, g and beta while staging each chunk, and the per-chunk
// launch applies the chain rule back to q, k, g and beta when it stores the
// token gradients (gdn_token_grads).
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace wkv7 {
namespace {

constexpr int kL = 16;                  // chunk length (= checkpoint interval)
constexpr float kMinChunkLogDecay = -60.0f;

// Packed sequences (cu == nullptr: the fixed-length form, in which
// n_state == 1 means one initial state shared by every sequence).  Sequence n owns
// tokens [cu[n], cu[n+1]) of the total_T-token axis, each offset clamped into
// range as the forward does; its checkpoints are chunks ck_off[n] ..
// ck_off[n+1] - 1 of the workspace (ck_off saturates at the capacity, so
// malformed offsets give wrong results, never an access out of bounds).
struct SeqGeom {
    const int32_t *cu = nullptr;
    const int32_t *ck_off = nullptr;
    const int32_t *smap = nullptr;
    int n_state = 0;
    int nseq = 0;
    int total_T = 0;
};

__device__ __forceinline__ void seq_range(const SeqGeom &vg, int n, int &tb, int &te)
{
    tb = min(max(vg.cu[n], 0), vg.total_T);
    te = min(max(vg.cu[n + 1], tb), vg.total_T);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc (16 x 16) += A (16 x KC) B (KC x 16), elements fetched by fa(m, kk)
// and fb(kk, n).  Lane l supplies A[l%16][kk0 + l/16] and B[kk0 + l/16][l%16]
// per step; the result lane l holds rows 4(l/16) .. +3 of column l%16.
template <int KC, class FA, class FB>
__device__ __forceinline__ f32x4 mm16(f32x4 acc, FA fa, FB fb, int lane)
{
    const int m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < KC; k0 += 4) acc = mfma_f32(fa(m, k0 + q), fb(k0 + q, m), acc);
    return acc;
}

// ---- launch 2: per-chunk gradients (and helpers shared with launch 1) --------

// Four consecutive elements (index i a multiple of 4) as fp32.
template <typename T> struct io4;
template <> struct io4<float> {
    __device__ __forceinline__ static f32x4 load(const float *p, size_t i) { return *(const f32x4 *)(p + i); }
    __device__ __forceinline__ static void store(float *p, size_t i, f32x4 x) { *(f32x4 *)(p + i) = x; }
};
template <> struct io4<uint16_t> {
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

// row_shl:n inside each 16-lane row (lane i reads lane i + n); lanes without
// a source receive `fill`.
template <int N>
__device__ __forceinline__ float row_shl(float x, float fill)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x100 + N, 0xF,
                                                      0xF, false));
}

// LDS of one chunk.  v and d_o stay in the I/O type (they are exact inputs),
// which at bf16 and D = 64 brings the total under 40 KB: four workgroups per
// CU.
template <int D, typename T_IO> struct alignas(16) GradLds {
    static constexpr int LD = D + 4;                  // fp32 tile rows (16-byte aligned)
    static constexpr int LDV = D + 16 / sizeof(T_IO); // I/O-type tile rows (16-byte aligned)
    float R[kL][LD], B[kL][LD], A[kL][LD], K[kL][LD];
    T_IO V[kL][LDV], DO[kL][LDV];
    float U[kL][LD];                    // X, then U (exact path: raw w)
    union {
        struct {
            float G[kL][LD];            // decay prefix
            float DX[kL][LD];           // dU, then dX
            // M_ba, then T in its place; M_bk, M_ra, M_rk; after the value
            // gradient, dM_ra, dM_rk, dM_ba, dM_bk in the same four slots
            float M[4][kL][kL + 1];
        };
        float RED[5][D / 16][D];        // exact path (which needs none of the above): per-wave row sums
    };
    float EGL[D];
    float gs[4][kL];                    // Gated DeltaNet: g, beta, 1/|q|, 1/|k| per token
    float gsum[5][2];                   // Gated DeltaNet exact path: per-wave channel sums
    int upd[kL];
};

enum { M_BA = 0, M_BK = 1, M_RA = 2, M_RK = 3, M_T = 0, DM_RA = 0, DM_RK = 1, DM_BA = 2, DM_BK = 3 };

// Element (row, col) of an I/O-type LDS tile as fp32, and four consecutive
// elements (col a multiple of 4).
__device__ __forceinline__ float tl(const float &x) { return x; }
__device__ __forceinline__ float tl(const uint16_t &x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ f32x4 tl4(const float *p) { return *(const f32x4 *)p; }
__device__ __forceinline__ f32x4 tl4(const uint16_t *p)
{
    const u32x2 u = *(const u32x2 *)p;
    return f32x4{bf16_lo(u[0]), bf16_hi(u[0]), bf16_lo(u[1]), bf16_hi(u[1])};
}

// Exact path: tokens of the chunk in reverse, each step's gradients from the
// per-token formulas (those of the oracle's derivative), with the states
// S_{t-1} and S_t recomputed from the chunk's checkpoint.  Lane layout of the
// recurrent kernel: lane (j, g) of wave w holds rows [g D/4, (g+1) D/4) of
// column 16w + j.  s.U holds the raw (masked) w.
template <int D, typename T_IO, bool GDN>
__device__ void chunk_grad_exact(GradLds<D, T_IO> &s, const float *Sc, const float *dSe, int Lc, size_t tokbase,
                                 int H, T_IO *dr, T_IO *dw, T_IO *dk, T_IO *dv, T_IO *da, T_IO *db)
{
    constexpr int RPL = D / 4, NW = D / 16;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = wave * 16 + (lane & 15), g = lane >> 4, row0 = g * RPL;
    auto colsum = [](float x) { return xsum32(xsum16(x)); };
    const auto &W = s.U;
    auto step = [&](float *P, int u) {   // P <- state after token u (P = state before it)
        if (!s.upd[u]) return;
        float sb = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) sb = fmaf(s.B[u][row0 + i], P[i], sb);
        sb = colsum(sb);
        const float vj = tl(s.V[u][col]);
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            P[i] = fmaf(__expf(W[u][row0 + i]), P[i], fmaf(s.A[u][row0 + i], sb, s.K[u][row0 + i] * vj));
    };
    auto rowsum = [&](float y, int e, int row) {   // over the 16 columns of the wave
        y += __shfl_xor(y, 1, kWave);
        y += __shfl_xor(y, 2, kWave);
        y += __shfl_xor(y, 4, kWave);
        y += __shfl_xor(y, 8, kWave);
        if ((lane & 15) == 0) s.RED[e][wave][row] = y;
    };
    float dS[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) dS[i] = dSe[(size_t)(row0 + i) * D + col];
    for (int t = Lc - 1; t >= 0; --t) {
        float P[RPL];   // S_{t-1}
#pragma unroll
        for (int i = 0; i < RPL; ++i) P[i] = Sc[(size_t)(row0 + i) * D + col];
        for (int u = 0; u < t; ++u) step(P, u);
        const bool up = s.upd[t] != 0;
        const float doj = tl(s.DO[t][col]), vj = tl(s.V[t][col]);
        float sb = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) sb = fmaf(s.B[t][row0 + i], P[i], sb);
        sb = colsum(sb);
        // dr_t = S_t d_o_t with S_t formed element by element from S_{t-1}
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const float st = up ? fmaf(__expf(W[t][row0 + i]), P[i], fmaf(s.A[t][row0 + i], sb, s.K[t][row0 + i] * vj))
                                : P[i];
            rowsum(st * doj, 0, row0 + i);
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i) dS[i] = fmaf(s.R[t][row0 + i], doj, dS[i]);
        float ad = 0.f, dvj = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            ad = fmaf(s.A[t][row0 + i], dS[i], ad);
            dvj = fmaf(s.K[t][row0 + i], dS[i], dvj);
        }
        ad = colsum(ad);
        dvj = colsum(dvj);
        if (g == 0) io<T_IO>::store(dv, tokbase + (size_t)t * H * D + col, up ? dvj : 0.0f);
        // row sums over this lane's column, then over the 16 columns of the
        // wave, then (through LDS) over the waves
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            rowsum(dS[i] * vj, 1, row0 + i);
            rowsum(dS[i] * sb, 2, row0 + i);
            rowsum(P[i] * ad, 3, row0 + i);
            rowsum(dS[i] * P[i], 4, row0 + i);
        }
        __syncthreads();
        float y[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
        if (tid < D) {
            for (int wv = 0; wv < NW; ++wv)
#pragma unroll
                for (int e = 0; e < 5; ++e) y[e] += s.RED[e][wv][tid];
        }
        const size_t gi = tokbase + (size_t)t * H * D + tid;
        if constexpr (GDN) {
            // the generalized-rule gradients of channel tid, then the chain
            // rule through the operands (see gdn_token_grads)
            const float gg = s.gs[0][t], bt = s.gs[1][t], eg = __expf(gg);
            const bool ch = tid < D;
            const int cc = ch ? tid : 0;   // channel of this thread (threads past D contribute zeros)
            const float gr = y[0], gk = up ? y[1] : 0.0f, ga = up ? y[2] : 0.0f, gb = up ? y[3] : 0.0f;
            const float gw = (up && ch) ? __expf(W[t][cc]) * y[4] : 0.0f;
            const float qn = ch ? s.R[t][cc] : 0.0f, kn = ch ? s.B[t][cc] : 0.0f;
            const float dkn = bt * gk - eg * bt * ga + gb;
            float pr[5] = {qn * gr, kn * dkn, kn * gk, kn * ga, gw};
#pragma unroll
            for (int e = 0; e < 5; ++e) {
#pragma unroll
                for (int msk = 1; msk < kWave; msk <<= 1) pr[e] += __shfl_xor(pr[e], msk, kWave);
            }
            if (lane == 0 && wave < D / kWave)
#pragma unroll
                for (int e = 0; e < 5; ++e) s.gsum[e][wave] = pr[e];
            __syncthreads();
            if (ch) {
                float S5[5];
#pragma unroll
                for (int e = 0; e < 5; ++e) S5[e] = D > kWave ? s.gsum[e][0] + s.gsum[e][1] : s.gsum[e][0];
                io<T_IO>::store(dr, gi, s.gs[2][t] * (gr - qn * S5[0]));   // dq
                io<T_IO>::store(dk, gi, s.gs[3][t] * (dkn - kn * S5[1]));
                if (tid == 0) {
                    const size_t si = tokbase / D + (size_t)t * H;
                    io<T_IO>::store(da, si, S5[2] - eg * S5[3]);             // dbeta
                    io<T_IO>::store(dw, si, S5[4] - eg * bt * S5[3]);        // dg
                }
            }
        } else if (tid < D) {
            io<T_IO>::store(dr, gi, y[0]);
            io<T_IO>::store(dk, gi, up ? y[1] : 0.0f);
            io<T_IO>::store(da, gi, up ? y[2] : 0.0f);
            io<T_IO>::store(db, gi, up ? y[3] : 0.0f);
            io<T_IO>::store(dw, gi, up ? __expf(W[t][tid]) * y[4] : 0.0f);
        }
        __syncthreads();
        if (up) {
#pragma unroll
            for (int i = 0; i < RPL; ++i)
                dS[i] = fmaf(__expf(W[t][row0 + i]), dS[i], s.B[t][row0 + i] * ad);
        }
    }
}

// Transposed product over a contraction of length D:
//   acc(16 x 16) += A (16 x D) B (D x 16) with A[m][j] = a4(m, j0) and
//   B[j][n] = b4(n, j0) fetched as four consecutive j = j0 .. j0 + 3.
// The contraction index is permuted inside each block of 16 so that in step
// s of block j0b lane (q, m) supplies j = j0b + 4q + s for both operands;
// this lets each lane feed four steps from one 16-byte load of a row.
template <int D, class FA, class FB>
__device__ __forceinline__ f32x4 mm16_rows(f32x4 acc, FA a4, FB b4, int lane)
{
    const int m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int j0b = 0; j0b < D; j0b += 16) {
        const f32x4 x = a4(m, j0b + 4 * q);
        const f32x4 y = b4(m, j0b + 4 * q);
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma_f32(x[st], y[st], acc);
    }
    return acc;
}

// Gated DeltaNet: the chain rule from the generalized-rule gradients of
// token t (lane (q, m) = (channel group, token): channels ch .. ch + 3) to
// the Gated DeltaNet inputs,
//   dkn = beta dk - e^g beta da + db,  dqn = dr,
//   dq = (dqn - qn (qn . dqn)) / |q|,  dk = (dkn - kn (kn . dkn)) / |k|,
//   dbeta = kn . dk - e^g kn . da,     dg = sum_c dw_c - e^g beta kn . da
// (|x| = sqrt(sum x^2 + 1e-6)).  The five channel sums are taken over the
// four lanes of the token in each wave, then across the waves through LDS
// (the dX tile, which every wave has finished with once all have passed the
// first barrier below).  qn and kn are the raw r and b operands.
template <int D, typename T_IO>
__device__ __forceinline__ void gdn_token_grads(GradLds<D, T_IO> &s, int t, int ch, int Lc, size_t tokbase, int H,
                                                f32x4 gr, f32x4 gw, f32x4 gk, f32x4 ga, f32x4 gb, f32x4 qn,
                                                f32x4 kn, T_IO *dq, T_IO *dg, T_IO *dk, T_IO *dbeta)
{
    constexpr int NW = D / 16;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, q = lane >> 4;
    const float gg = s.gs[0][t], bt = s.gs[1][t], eg = __expf(gg);
    const f32x4 dkn = gk * bt - ga * (eg * bt) + gb;
    float pr[5] = {dot4(qn, gr), dot4(kn, dkn), dot4(kn, gk), dot4(kn, ga), gw[0] + gw[1] + gw[2] + gw[3]};
#pragma unroll
    for (int e = 0; e < 5; ++e) pr[e] = xsum32(xsum16(pr[e]));
    __syncthreads();
    float(*red)[NW][kL] = reinterpret_cast<float(*)[NW][kL]>(&s.DX[0][0]);
    static_assert(sizeof(float) * 5 * NW * kL <= sizeof(s.DX), "reduction fits the dX tile");
    if (q == 0)
#pragma unroll
        for (int e = 0; e < 5; ++e) red[e][wave][t] = pr[e];
    __syncthreads();
    float S5[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 5; ++e)
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) S5[e] += red[e][wv][t];
    if (t < Lc) {
        const size_t gi = tokbase + (size_t)t * H * D + ch;
        io4<T_IO>::store(dq, gi, (gr - qn * S5[0]) * s.gs[2][t]);
        io4<T_IO>::store(dk, gi, (dkn - kn * S5[1]) * s.gs[3][t]);
        if (wave == 0 && q == 0) {
            const size_t si = tokbase / D + (size_t)t * H;
            io<T_IO>::store(dbeta, si, S5[2] - eg * S5[3]);
            io<T_IO>::store(dg, si, S5[4] - eg * bt * S5[3]);
        }
    }
}

// One workgroup per (b, h, chunk), D/16 waves.
// At D = 64 with bf16 I/O, 40 000 bytes of LDS and at most 128 VGPRs hold
// four workgroups on a CU (the whole backward at B8 T4096 H64 measured
// 5.82 -> 5.26 ms against three).  At D = 128 the same register limit spills, and a second
// workgroup per CU would also push the second pass over the checkpoint and
// the end gradient out of L2 (measured slower), so that size keeps one.
template <int D, typename T_IO, bool GDN>
__global__ __launch_bounds__(D * 4) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 1))) void chunk_grad_kernel(
    int T, int H, int nck, const T_IO *__restrict__ r, const T_IO *__restrict__ w,
    const T_IO *__restrict__ k, const T_IO *__restrict__ v, const T_IO *__restrict__ a,
    const T_IO *__restrict__ b, const uint8_t *__restrict__ mask, const T_IO *__restrict__ d_o,
    const float *__restrict__ ckpt, const float *__restrict__ dck, T_IO *__restrict__ dr,
    T_IO *__restrict__ dw, T_IO *__restrict__ dk, T_IO *__restrict__ dv, T_IO *__restrict__ da,
    T_IO *__restrict__ db, SeqGeom vg)
{
    constexpr int NT = D * 4;
    using Lds = GradLds<D, T_IO>;
    __shared__ Lds s;
    // chunk c of sequence n, head h; tokens from tok0 (packed: the sequence's
    // first token; fixed-length: n T), checkpoint index ckid
    int n, h, c, Tn;
    size_t tok0, ckid;
    if (vg.cu) {
        const int gc = (int)(blockIdx.x / H);
        h = (int)(blockIdx.x % H);
        if (gc >= vg.ck_off[vg.nseq]) return;   // the whole workgroup, before any barrier
        // the sequence owning global chunk gc: the last n with ck_off[n] <= gc
        int lo = 0, hi = vg.nseq;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (vg.ck_off[mid] <= gc) lo = mid;
            else hi = mid;
        }
        n = lo;
        c = gc - vg.ck_off[n];
        int tb, te;
        seq_range(vg, n, tb, te);
        tok0 = (size_t)tb;
        Tn = te - tb;
        ckid = (size_t)gc * H + h;
    } else {
        const int bh0 = (int)(blockIdx.x / nck);
        c = (int)(blockIdx.x % nck);
        n = bh0 / H;
        h = bh0 % H;
        tok0 = (size_t)n * T;
        Tn = T;
        ckid = (size_t)bh0 * nck + c;
    }
    const int t0 = c * kL, Lc = min(kL, Tn - t0);
    const size_t tokbase = ((tok0 + t0) * H + h) * D;   // element of (token t0, channel 0)
    const float *Sc = ckpt + ckid * D * D;
    const float *dSe = dck + ckid * D * D;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int q = lane >> 4, m = lane & 15;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    // At D = 64 with bf16 I/O the state and dS' values of the value-column
    // products, and the rows of S and dS' for the key-channel products, are
    // loaded into registers first, so that their latency overlaps the
    // staging and chunk-matrix phases and both reads of each line come close
    // together (measured 8 % faster, despite about 32 spilled registers; at
    // D = 128, or with fp32 I/O, the extra registers cost occupancy).  Lane
    // (q, m) holds rows 16 jb + 4 q + st, column 16 wave + m, at index
    // 4 jb + st: the contraction order in which each lane reads the other
    // operand as one 16-byte row segment per four MFMA steps.
    constexpr bool kPre = D == 64 && sizeof(T_IO) == 2;
    float scol[D / 4], dcol[D / 4];
    if constexpr (kPre) {
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
            const size_t e = (size_t)(16 * (i >> 2) + 4 * q + (i & 3)) * D + 16 * wave + m;
            scol[i] = Sc[e];
            dcol[i] = dSe[e];
        }
    }
    f32x4 srow[D / 16], drow[D / 16];
    if constexpr (kPre) {
        const size_t rowp = (size_t)(16 * wave + m) * D + 4 * q;
#pragma unroll
        for (int jb = 0; jb < D / 16; ++jb) {
            srow[jb] = *(const f32x4 *)(Sc + rowp + 16 * jb);
            drow[jb] = *(const f32x4 *)(dSe + rowp + 16 * jb);
        }
    }

    // raw inputs of the chunk, four channels per thread; a token that does
    // not update gets w = k = a = b = 0 and v = 0 (an exact identity step),
    // tokens past T are all zero.  The loads carry no condition (a token
    // past the chunk's end reads the chunk's last token, then takes zeros)
    // and the mask byte is applied afterwards, so that they are all in
    // flight together.
    {
        static_assert(NT == kL * D / 4, "one thread per (token, 4 channels)");
        const int t = tid / (D / 4), c4 = 4 * (tid % (D / 4));
        const bool valid = t < Lc;
        const size_t gi = tokbase + (size_t)min(t, Lc - 1) * H * D + c4;
        using R4 = raw4<T_IO>;
        if constexpr (GDN) {
            const size_t si = tokbase / D + (size_t)min(t, Lc - 1) * H;
            const typename R4::type do4 = R4::load(d_o, gi), v4 = R4::load(v, gi);
            const f32x4 q4l = io4<T_IO>::load(r, gi), k4l = io4<T_IO>::load(k, gi);
            const float ggl = io<T_IO>::load(w, si), btl = io<T_IO>::load(a, si);
            const f32x4 q4 = valid ? q4l : z, k4 = valid ? k4l : z;
            const float gg = valid ? ggl : 0.0f, bt = valid ? btl : 0.0f;
            *(typename R4::type *)&s.DO[t][c4] = valid ? do4 : R4::zero();
            *(typename R4::type *)&s.V[t][c4] = valid ? v4 : R4::zero();
            const float iq = inv_norm<D>(q4), ik = inv_norm<D>(k4);
            const f32x4 kn = k4 * ik;
            *(f32x4 *)&s.R[t][c4] = q4 * iq;
            *(f32x4 *)&s.G[t][c4] = f32x4{gg, gg, gg, gg};
            *(f32x4 *)&s.K[t][c4] = kn * bt;
            *(f32x4 *)&s.A[t][c4] = kn * (-__expf(gg) * bt);
            *(f32x4 *)&s.B[t][c4] = kn;
            if (c4 == 0) {
                s.gs[0][t] = gg;
                s.gs[1][t] = bt;
                s.gs[2][t] = iq;
                s.gs[3][t] = ik;
                s.upd[t] = valid;
            }
        } else {
            int mb = 1;
            if (mask) mb = mask[tok0 + t0 + min(t, Lc - 1)];
            const typename R4::type do4 = R4::load(d_o, gi), v4 = R4::load(v, gi);
            const f32x4 r4 = io4<T_IO>::load(r, gi), w4 = io4<T_IO>::load(w, gi);
            const f32x4 k4 = io4<T_IO>::load(k, gi), a4 = io4<T_IO>::load(a, gi);
            const f32x4 b4 = io4<T_IO>::load(b, gi);
            // (an empty asm keeps the compare of the mask byte after the loads)
            asm volatile("" : "+v"(mb));
            const bool up = valid && mb != 0;
            *(typename R4::type *)&s.DO[t][c4] = valid ? do4 : R4::zero();
            *(typename R4::type *)&s.V[t][c4] = up ? v4 : R4::zero();
            *(f32x4 *)&s.R[t][c4] = valid ? r4 : z;
            *(f32x4 *)&s.G[t][c4] = up ? w4 : z;
            *(f32x4 *)&s.K[t][c4] = up ? k4 : z;
            *(f32x4 *)&s.A[t][c4] = up ? a4 : z;
            *(f32x4 *)&s.B[t][c4] = up ? b4 : z;
            if (c4 == 0) s.upd[t] = up;
        }
    }
    __syncthreads();
    int extreme = 0;
    if (tid < D) {
        float x[kL];
#pragma unroll
        for (int t = 0; t < kL; ++t) x[t] = s.G[t][tid];
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < kL; ++t) {
            extreme |= x[t] > 0.0f;
            acc += x[t];
            s.G[t][tid] = acc;
        }
        extreme |= acc < kMinChunkLogDecay;
        s.EGL[tid] = __expf(acc);
    }
    if (__syncthreads_or(extreme)) {
        // raw w for the exact path (the prefix replaced it in G)
        {
            const int t = tid / (D / 4), c4 = 4 * (tid % (D / 4));
            const size_t gi = tokbase + (size_t)t * H * D + c4;
            if constexpr (GDN) {
                const float gg = s.gs[0][t];
                *(f32x4 *)&s.U[t][c4] = s.upd[t] ? f32x4{gg, gg, gg, gg} : z;
            } else {
                *(f32x4 *)&s.U[t][c4] = s.upd[t] ? io4<T_IO>::load(w, gi) : z;
            }
        }
        __syncthreads();
        chunk_grad_exact<D, T_IO, GDN>(s, Sc, dSe, Lc, tokbase, H, dr, dw, dk, dv, da, db);
        return;
    }
    {
        const int t = tid / (D / 4), c4 = 4 * (tid % (D / 4));
        const f32x4 G = *(const f32x4 *)&s.G[t][c4];
        const f32x4 Gp = t ? *(const f32x4 *)&s.G[t - 1][c4] : z;
        f32x4 eG, enG, eGp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            eG[i] = __expf(G[i]);
            enG[i] = __expf(-G[i]);
            eGp[i] = __expf(Gp[i]);
        }
        *(f32x4 *)&s.R[t][c4] *= eG;
        *(f32x4 *)&s.B[t][c4] *= eGp;
        *(f32x4 *)&s.A[t][c4] *= enG;
        *(f32x4 *)&s.K[t][c4] *= enG;
    }
    __syncthreads();
    // chunk matrices
    if (wave < 4) {
        const float(*X)[Lds::LD] = wave < 2 ? s.B : s.R;
        const float(*Y)[Lds::LD] = (wave & 1) ? s.K : s.A;
        const f32x4 acc = mm16_rows<D>(z, [&](int mm, int j) { return *(const f32x4 *)&X[mm][j]; },
                                       [&](int n, int j) { return *(const f32x4 *)&Y[n][j]; }, lane);
        const bool strict = wave < 2;   // M_ba, M_bk strictly lower; M_ra, M_rk with the diagonal
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * q + i;
            s.M[wave][row][m] = (strict ? row > m : row >= m) ? acc[i] : 0.0f;
        }
    }
    __syncthreads();
    // T = (I - M_ba)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8) (N = M_ba
    // strictly lower, N^16 = 0), formed by wave 0 on the matrix cores as in
    // the chain kernel (acc(X Y) = sum_st mfma(acc(X^T)[st], acc(Y)[st])) and
    // written over M_ba row-major.  The wave reads all of M_ba before it
    // writes.
    if (wave == 0) {
        auto mm = [](f32x4 aT, f32x4 b) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) c = mfma_f32(aT[st], b[st], c);
            return c;
        };
        f32x4 nA, nT, eye;   // acc(N), acc(N^T), I
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            nA[i] = s.M[M_BA][4 * q + i][m];
            nT[i] = s.M[M_BA][m][4 * q + i];
            eye[i] = 4 * q + i == m ? 1.0f : 0.0f;
        }
        const f32x4 n2 = mm(nT, nA), n2T = mm(nA, nT);
        const f32x4 n4 = mm(n2T, n2), n4T = mm(n2, n2T);
        const f32x4 n8 = mm(n4T, n4);
        const f32x4 p1T = mm(eye + n2, eye + nT);   // ((I + N)(I + N^2))^T
        const f32x4 p2T = mm(eye + n4, p1T);        // (P1 (I + N^4))^T
        const f32x4 tA = mm(p2T, eye + n8);         // acc(T)
#pragma unroll
        for (int i = 0; i < 4; ++i) s.M[M_T][4 * q + i][m] = tA[i];
    }
    __syncthreads();

    // --- value-column slice c0 .. c0 + 15 of this wave ---
    const int c0 = 16 * wave;
    auto dY = [&](int kk, int n) { return s.EGL[kk] * dSe[(size_t)kk * D + c0 + n]; };
    {
        f32x4 X = z;
        if constexpr (kPre) {
#pragma unroll
            for (int jb = 0; jb < D / 16; ++jb) {
                const f32x4 bt = *(const f32x4 *)&s.B[m][16 * jb + 4 * q];
#pragma unroll
                for (int st = 0; st < 4; ++st) X = mfma_f32(bt[st], scol[4 * jb + st], X);
            }
        } else {
            X = mm16<D>(z, [&](int mm, int kk) { return s.B[mm][kk]; },
                        [&](int kk, int n) { return Sc[(size_t)kk * D + c0 + n]; }, lane);
        }
        X = mm16<kL>(X, [&](int mm, int kk) { return s.M[M_BK][mm][kk]; },
                     [&](int kk, int n) { return tl(s.V[kk][c0 + n]); }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) s.U[4 * q + i][c0 + m] = X[i];
    }
    f32x4 dU = z;
    if constexpr (kPre) {
#pragma unroll
        for (int jb = 0; jb < D / 16; ++jb) {
            const f32x4 at = *(const f32x4 *)&s.A[m][16 * jb + 4 * q], eg = *(const f32x4 *)&s.EGL[16 * jb + 4 * q];
#pragma unroll
            for (int st = 0; st < 4; ++st) dU = mfma_f32(at[st], eg[st] * dcol[4 * jb + st], dU);
        }
    } else {
        dU = mm16<D>(z, [&](int mm, int kk) { return s.A[mm][kk]; }, dY, lane);
    }
    dU = mm16<kL>(dU, [&](int mm, int kk) { return s.M[M_RA][kk][mm]; },
                  [&](int kk, int n) { return tl(s.DO[kk][c0 + n]); }, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) s.DX[4 * q + i][c0 + m] = dU[i];
    __syncthreads();
    {
        // this wave alone reads and writes columns c0 .. c0 + 15 of U and DX
        const f32x4 U = mm16<kL>(z, [&](int mm, int kk) { return s.M[M_T][mm][kk]; },
                                 [&](int kk, int n) { return s.U[kk][c0 + n]; }, lane);
        const f32x4 dX = mm16<kL>(z, [&](int mm, int kk) { return s.M[M_T][kk][mm]; },
                                  [&](int kk, int n) { return s.DX[kk][c0 + n]; }, lane);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s.U[4 * q + i][c0 + m] = U[i];
            s.DX[4 * q + i][c0 + m] = dX[i];
        }
    }
    __syncthreads();
    {
        // dV = K^ dY + M_rk^T dO + M_bk^T dX, formed transposed (value columns
        // c0 + 4q + i of token m in lane (q, m)) so that each lane stores four
        // adjacent columns
        f32x4 dVt = z;
        if constexpr (kPre) {
#pragma unroll
            for (int jb = 0; jb < D / 16; ++jb) {
                const f32x4 kt = *(const f32x4 *)&s.K[m][16 * jb + 4 * q], eg = *(const f32x4 *)&s.EGL[16 * jb + 4 * q];
#pragma unroll
                for (int st = 0; st < 4; ++st) dVt = mfma_f32(eg[st] * dcol[4 * jb + st], kt[st], dVt);
            }
        } else {
            dVt = mm16<D>(z, [&](int mm, int kk) { return dY(kk, mm); },
                          [&](int kk, int n) { return s.K[n][kk]; }, lane);
        }
        dVt = mm16<kL>(dVt, [&](int mm, int kk) { return tl(s.DO[kk][c0 + mm]); },
                       [&](int kk, int n) { return s.M[M_RK][kk][n]; }, lane);
        dVt = mm16<kL>(dVt, [&](int mm, int kk) { return s.DX[kk][c0 + mm]; },
                       [&](int kk, int n) { return s.M[M_BK][kk][n]; }, lane);
        if (m < Lc) io4<T_IO>::store(dv, tokbase + (size_t)m * H * D + c0 + 4 * q, s.upd[m] ? dVt : z);
    }
    // --- gradients of the chunk matrices (contractions over the value columns):
    // wave 0 dM_ra = dO U^T, wave 1 dM_rk = dO V^T, wave 2 dM_ba = dX U^T,
    // wave 3 dM_bk = dX V^T; stored over the chunk matrices once every wave
    // is past the value gradient ---
    f32x4 dmacc = z;
    {
        auto rowDO = [&](int mm, int j) { return tl4(&s.DO[mm][j]); };
        auto rowDX = [&](int mm, int j) { return *(const f32x4 *)&s.DX[mm][j]; };
        auto rowU = [&](int n, int j) { return *(const f32x4 *)&s.U[n][j]; };
        auto rowV = [&](int n, int j) { return tl4(&s.V[n][j]); };
        if (wave == 0) dmacc = mm16_rows<D>(z, rowDO, rowU, lane);
        else if (wave == 1) dmacc = mm16_rows<D>(z, rowDO, rowV, lane);
        else if (wave == 2) dmacc = mm16_rows<D>(z, rowDX, rowU, lane);
        else if (wave == 3) dmacc = mm16_rows<D>(z, rowDX, rowV, lane);
    }
    __syncthreads();
    if (wave < 4) {
        const bool strict = wave >= 2;   // dM_ba, dM_bk strictly lower
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * q + i;
            s.M[DM_RA + wave][row][m] = (strict ? row > m : row >= m) ? dmacc[i] : 0.0f;
        }
    }
    __syncthreads();

    // --- key-channel slice k0 .. k0 + 15 of this wave, as transposed tiles:
    // lane (q, m) ends with channels k0 + 4q + i of token m ---
    const int k0 = 16 * wave;
    const size_t rowm = (size_t)(k0 + m) * D;   // state row of channel k0 + m
    // The four products that contract over the value columns, with each row
    // of S and dS' loaded once (the contraction index is permuted as in
    // mm16_rows): dR~^T += S dO^T, dB~^T += S dX^T, dA^^T += dY U^T,
    // dK^^T += dY V^T.  sds collects sum_j dS'[k0+m][j] S[k0+m][j].
    f32x4 dR = z, dB = z, dA = z, dK = z;
    float sds = 0.0f;
    {
        const float eglm = s.EGL[k0 + m];
#pragma unroll
        for (int j0b = 0; j0b < D; j0b += 16) {
            const int j = j0b + 4 * q;
            f32x4 sr, dr4;
            if constexpr (kPre) {
                sr = srow[j0b / 16];
                dr4 = drow[j0b / 16];
            } else {
                sr = *(const f32x4 *)(Sc + rowm + j);
                dr4 = *(const f32x4 *)(dSe + rowm + j);
            }
            sds += dr4[0] * sr[0] + dr4[1] * sr[1] + dr4[2] * sr[2] + dr4[3] * sr[3];
            const f32x4 dy = dr4 * eglm;
            const f32x4 yo = tl4(&s.DO[m][j]), yx = *(const f32x4 *)&s.DX[m][j];
            const f32x4 yu = *(const f32x4 *)&s.U[m][j], yv = tl4(&s.V[m][j]);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                dR = mfma_f32(sr[st], yo[st], dR);
                dB = mfma_f32(sr[st], yx[st], dB);
                dA = mfma_f32(dy[st], yu[st], dA);
                dK = mfma_f32(dy[st], yv[st], dK);
            }
        }
    }
    sds = xsum32(xsum16(sds));   // channel k0 + m, in every lane of column m
    // Chunk-end term of dw, sum_j dS'[c][j] S'[c][j] with S' = diag(e^{G_L})
    // (S + A^^T U + K^^T V): e^{G_L,c} sds_c + sum_t A^[t][c] (U dY^T)[t][c]
    // + sum_t K^[t][c] (V dY^T)[t][c]; the last two sums run over this row's
    // 16 lanes (tokens), with dA and dK still holding only those products.
    float dglc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = k0 + 4 * q + i;
        float y = s.A[m][c] * dA[i] + s.K[m][c] * dK[i];
        y += __shfl_xor(y, 1, kWave);
        y += __shfl_xor(y, 2, kWave);
        y += __shfl_xor(y, 4, kWave);
        y += __shfl_xor(y, 8, kWave);
        dglc[i] = s.EGL[c] * __shfl(sds, 4 * q + i, 16) + y;
    }
    // small terms: (dM X)^T = X^T dM^T and (dM^T X)^T = X^T dM
    auto colT = [&](const float(*X)[Lds::LD]) { return [X, k0](int mm, int kk) { return X[kk][k0 + mm]; }; };
    auto dMt = [&](int idx) { return [idx](int kk, int n) { return s.M[idx][n][kk]; }; };
    auto dMn = [&](int idx) { return [idx](int kk, int n) { return s.M[idx][kk][n]; }; };
    dR = mm16<kL>(dR, colT(s.A), dMt(DM_RA), lane);
    dR = mm16<kL>(dR, colT(s.K), dMt(DM_RK), lane);
    dB = mm16<kL>(dB, colT(s.A), dMt(DM_BA), lane);
    dB = mm16<kL>(dB, colT(s.K), dMt(DM_BK), lane);
    dA = mm16<kL>(dA, colT(s.R), dMn(DM_RA), lane);
    dA = mm16<kL>(dA, colT(s.B), dMn(DM_BA), lane);
    dK = mm16<kL>(dK, colT(s.R), dMn(DM_RK), lane);
    dK = mm16<kL>(dK, colT(s.B), dMn(DM_BK), lane);

    // token gradients of token t = m, channels ch = k0 + 4q .. + 3
    const int t = m, ch = k0 + 4 * q;
    const f32x4 G = *(const f32x4 *)&s.G[t][ch];
    const f32x4 Gp = t ? *(const f32x4 *)&s.G[t - 1][ch] : z;
    const f32x4 Rs = *(const f32x4 *)&s.R[t][ch], Bs = *(const f32x4 *)&s.B[t][ch];
    const f32x4 As = *(const f32x4 *)&s.A[t][ch], Ks = *(const f32x4 *)&s.K[t][ch];
    f32x4 gr, gb, ga, gk, gw, rraw, braw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float eG = __expf(G[i]), enG = __expf(-G[i]), eGp = __expf(Gp[i]);
        gr[i] = dR[i] * eG;
        gb[i] = dB[i] * eGp;
        ga[i] = dA[i] * enG;
        gk[i] = dK[i] * enG;
        // raw (masked) operands are the scaled ones times the inverse factors
        const float rr = Rs[i] * enG, kk = Ks[i] * eG, aa = As[i] * eG, bv = Bs[i] * __expf(-Gp[i]);
        rraw[i] = rr;
        braw[i] = bv;
        const float p = gr[i] * rr - ga[i] * aa - gk[i] * kk;
        const float qb = gb[i] * bv;
        // dG_t = p_t + qb_{t+1} (+ the chunk-end term at t = 15), then the
        // suffix sum over t = m .. 15 within the 16-lane row
        float y = p + row_shl<1>(qb, 0.0f) + (t == kL - 1 ? dglc[i] : 0.0f);
        y += row_shl<1>(y, 0.0f);
        y += row_shl<2>(y, 0.0f);
        y += row_shl<4>(y, 0.0f);
        y += row_shl<8>(y, 0.0f);
        gw[i] = y;
    }
    if constexpr (GDN) {
        gdn_token_grads<D, T_IO>(s, t, ch, Lc, tokbase, H, gr, gw, gk, ga, gb, rraw, braw, dr, dw, dk, da);
    } else if (t < Lc) {
        const bool up = s.upd[t] != 0;
        const size_t gi = tokbase + (size_t)t * H * D + ch;
        io4<T_IO>::store(dr, gi, gr);
        io4<T_IO>::store(dw, gi, up ? gw : z);
        io4<T_IO>::store(dk, gi, up ? gk : z);
        io4<T_IO>::store(da, gi, up ? ga : z);
        io4<T_IO>::store(db, gi, up ? gb : z);
    }
}

// ---- launch 1: the two recurrences in chunk form -------------------------------

// Value columns of the state are independent in both recurrences (column j
// of S' reads only column j of S, and the same holds for dS), so a sequence's
// state is split over workgroups of four waves and 64 columns (kChainCols);
// each workgroup forms the chunk's token-by-token matrices itself.
constexpr int kChainWaves = 4;
constexpr int kChainCols = 16 * kChainWaves;

// LDS of one chunk: under 40 KB at D = 128 with bf16 I/O, so four workgroups
// share a CU.  v and d_o (this workgroup's columns only) stay in the I/O
// type; the chunk matrices and T take the place of the decay prefix once
// the operands are scaled.
template <int D, typename T_IO> struct alignas(16) ChainLds {
    static constexpr int LD = D + 4;                             // fp32 tile rows (16-byte aligned)
    static constexpr int LDY = kChainCols + 16 / sizeof(T_IO);   // I/O-type tile rows (16-byte aligned)
    union {
        float G[kL][LD];                // w, then its decay prefix (exact path: raw w again)
        // after the scaling: the chunk matrices as two partial sums each
        // (the two halves of the channel contraction): M[half] M_ba,
        // M[2 + half] M_ba transposed, M[4 + half] M_bk (forward) or M_ra
        // (backward)
        float M[6][kL][20];
    };
    float A[kL][LD];                    // a, then A^ = a e^{-G}
    float B[kL][LD];                    // b, then B~ = b e^{G_{t-1}}
    float X[kL][LD];                    // forward: k, then K^ = k e^{-G}; backward: r, then R~ = r e^G
    T_IO Y[kL][LDY];                    // forward: v; backward: d_o (this workgroup's columns)
    float EGL[D];
    int upd[kL];
};

// Store a state slice held as St[ti][i] = S[16 ti + 4q + i][col] (lane (q, m))
// into a row-major D x D matrix at dst (the same address in every lane),
// through one running 32-bit byte offset (a separate address per row would
// stay live across the chunk loop).
template <int D>
__device__ __forceinline__ void store_slice(float *dst, const f32x4 *St, int q, int col)
{
    unsigned off = (unsigned)(4 * q * D + col) * 4u;
#pragma unroll
    for (int ti = 0; ti < D / 16; ++ti)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(float *)((char *)dst + off) = St[ti][i];
            off += (i == 3) ? 13 * D * 4 : D * 4;
            asm volatile("" : "+v"(off));
        }
}

// Workgroups for the 2 nbh (role, sequence-head) pairs x D / 64 column
// groups.  Role 0 (forward) runs the forward recurrence chunk by chunk,
//   X = B~ S + M_bk V,  U = T X,  S <- diag(e^{G_L}) (S + A^T U + K^T V),
// storing the state before every 16-token chunk (ckpt[bh][c]); role 1
// runs the state-gradient recurrence backwards, with dS' the gradient at
// the chunk's end,
//   dY = diag(e^{G_L}) dS',  dU = A^ dY + M_ra^T dO,  dX = T^T dU,
//   dS <- dY + R~^T dO + B~^T dX,
// storing dS' of every chunk first (dck[bh][c]).  Wave w keeps columns
// col = 64 g + 16 w + m of its group g in MFMA accumulator layout,
// St[ti][i] = row 16 ti + 4q + i, for lane (q, m).  In every product that
// contracts over the state's rows or over the chunk's tokens, the
// contraction index is taken in the order the accumulator layout holds it
// (step st of tile ti takes rows 16 ti + 4q + st), so the state and the
// intermediate tiles feed the matrix cores straight from registers.  A chunk
// with a positive w, or whose decay reaches e^{-60}, runs token by token.
// Workgroup numbering: blocks of eight consecutive (role, bh) pairs, each
// block once per column group, so that the groups of one pair are eight
// workgroups apart (the same XCD, whose L2 then serves the chunk inputs that
// both read) and are dispatched together.  Four waves of at most 128 VGPRs
// and under 40 KB of LDS: four workgroups per CU, so that each CU
// interleaves the serial phases of one chunk (prefix, chunk matrices, T)
// with the matrix-core products of others.
template <int D, typename T_IO, bool GDN, bool ORDERED>
__global__ __launch_bounds__(kChainWaves * kWave) __attribute__((amdgpu_waves_per_eu(4))) void chain_kernel(
    int T, int H, int nbh, const T_IO *__restrict__ r, const T_IO *__restrict__ w,
    const T_IO *__restrict__ k, const T_IO *__restrict__ v, const T_IO *__restrict__ a,
    const T_IO *__restrict__ b, const float *__restrict__ s0, const uint8_t *__restrict__ mask,
    const T_IO *__restrict__ d_o, const float *__restrict__ d_sf, float *__restrict__ ckpt,
    float *__restrict__ dck, float *__restrict__ d_s0, SeqGeom vg)
{
    constexpr int NTILE = D / 16;                    // row tiles of the state
    constexpr int NCG = D / kChainCols;              // column groups
    constexpr int NT = kChainWaves * kWave;
    constexpr int NU = kL * (D / 4) / NT;            // staging units (token, 4 channels) per thread
    static_assert(NCG >= 1 && NU >= 1 && NU * NT == kL * (D / 4), "chunk tiles split evenly");
    static_assert(kL * kChainCols / 4 == NT, "one thread per (token, 4 columns) of the value tile");
    using Lds = ChainLds<D, T_IO>;
    __shared__ Lds s;
    const int pair = (int)(blockIdx.x / (8 * NCG)) * 8 + (int)(blockIdx.x % 8);
    const int cg = (int)(blockIdx.x / 8) % NCG;
    if (pair >= 2 * nbh) return;   // the whole workgroup, before any barrier
    const bool fwd = pair < nbh;
    const int bh = fwd ? pair : pair - nbh;
    const int h = bh % H;   // head
    // sequence: packed batches of few sequences run longest first (slot bh
    // takes the sequence of rank bh / H by length; ORDERED is chosen on the
    // host, use_longest_first)
    int bb = bh / H, lf_tb = 0, lf_te = 0;
    if constexpr (ORDERED) {
        __shared__ int lf_beg[kLongestFirstMax], lf_len[kLongestFirstMax], lf_rank[kLongestFirstMax], lf_pick[1];
        longest_first<1>(vg.cu, vg.total_T, vg.nseq, bh, H, lf_beg, lf_len, lf_rank, lf_pick);
        bb = lf_pick[0];
        lf_tb = lf_beg[bb];
        lf_te = lf_tb + lf_len[bb];
    }
    const int tid0 = threadIdx.x, wave = tid0 / kWave;
    const int q0 = (tid0 % kWave) >> 4, m0 = tid0 & 15;
    const int cw = kChainCols * cg + 16 * wave;   // this wave's first column
    const size_t st = (size_t)(ORDERED ? bb * H + h : bh) * D * D;   // this (sequence, head) in [B,H,D,D] arrays
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    // tokens tok0 .. tok0 + T - 1; chunk c's checkpoints at index ckidx(c),
    // stored for c < nck_store (fewer than the chunks only for malformed
    // packed offsets); initial state s0p (nullptr: zeros)
    size_t tok0, ck0;
    int nck_store;
    const float *s0p = nullptr;
    if (vg.cu) {
        int tb = lf_tb, te = lf_te;   // ORDERED: clamped by longest_first
        if (!ORDERED) seq_range(vg, bb, tb, te);
        tok0 = (size_t)tb;
        T = te - tb;
        ck0 = (size_t)vg.ck_off[bb];
        nck_store = vg.ck_off[bb + 1] - vg.ck_off[bb];
        if (s0) {
            // pool row: state_map[n]; without a map row n, or row 0 when the
            // pool holds one state shared by every sequence
            const int srow = vg.smap ? vg.smap[bb] : (vg.n_state == 1 ? 0 : bb);
            if (srow >= 0 && srow < vg.n_state) s0p = s0 + ((size_t)srow * H + h) * D * D;
        }
    } else {
        tok0 = (size_t)bb * T;
        ck0 = (size_t)bh * ((T + kL - 1) / kL);
        nck_store = (T + kL - 1) / kL;
        // one initial state shared by every sequence: row 0 of the pool
        if (s0) s0p = vg.n_state == 1 ? s0 + (size_t)h * D * D : s0 + st;
    }
    const int nck = (T + kL - 1) / kL;
    auto ckidx = [&](int c) { return vg.cu ? (ck0 + c) * H + h : ck0 + c; };

    f32x4 St[NTILE];
    {
        const float *init = fwd ? s0p : (d_sf ? d_sf + st : nullptr);
#pragma unroll
        for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
            for (int i = 0; i < 4; ++i) St[ti][i] = init ? init[(size_t)(16 * ti + 4 * q0 + i) * D + cw + m0] : 0.0f;
    }
    // the initial state is complete before the chunk loop (otherwise every
    // iteration's first checkpoint store would wait for all memory in flight)
#pragma unroll
    for (int ti = 0; ti < NTILE; ++ti)
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(St[ti][i]));
    // staging unit j of thread tid: token tpj, channels cpj .. cpj + 3 (the
    // D/4 threads of a token are adjacent lanes of one wave); value tile:
    // token tid / 16, columns 64 g + 4 (tid % 16) .. + 3
    auto tpj = [](int tid, int j) { return (tid + NT * j) / (D / 4); };
    auto cpj = [](int tid, int j) { return 4 * ((tid + NT * j) % (D / 4)); };
    using R4 = raw4<T_IO>;
    typename R4::type pf[NU][4], py;
    int pm[NU], pmy;
    float pg[NU], pb[NU];   // Gated DeltaNet: g and beta of the token
    const T_IO *const x_src = fwd ? k : r, *const y_src = fwd ? v : d_o;
    // Global addresses: a base common to the workgroup (the chunk's first
    // token, this head) plus a 32-bit per-lane byte offset.
    auto ld4 = [](const T_IO *base, unsigned e) {
        return *(const typename R4::type *)((const char *)base + e * (unsigned)sizeof(T_IO));
    };
    auto ld1 = [](const T_IO *base, unsigned e) {
        return io<T_IO>::load((const T_IO *)((const char *)base + e * (unsigned)sizeof(T_IO)), 0);
    };
    auto fetch = [&](int c, int tid) {
        const int t0 = c * kL, nt = min(kL, T - t0);
        const size_t cb = ((tok0 + t0) * H + h) * D;   // (token t0, channel 0)
        const size_t sb = (tok0 + t0) * H + h;         // Gated DeltaNet: per-token values
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int tp = tpj(tid, j);
            const bool valid = tp < nt;
            const unsigned gi = (unsigned)(tp * H * D + cpj(tid, j));
            if constexpr (GDN) {
                // k, then q (backward); every token updates
                const unsigned si = (unsigned)(tp * H);
                pf[j][0] = valid ? ld4(k + cb, gi) : R4::zero();
                pf[j][1] = (valid && !fwd) ? ld4(r + cb, gi) : R4::zero();
                pg[j] = valid ? ld1(w + sb, si) : 0.0f;
                pb[j] = valid ? ld1(a + sb, si) : 0.0f;
                pm[j] = valid;
            } else {
                // every valid token is loaded; the mask byte is applied when
                // the tiles are staged, so that no load waits for it
                pf[j][0] = valid ? ld4(w + cb, gi) : R4::zero();
                pf[j][1] = valid ? ld4(a + cb, gi) : R4::zero();
                pf[j][2] = valid ? ld4(b + cb, gi) : R4::zero();
                pf[j][3] = valid ? ld4(x_src + cb, gi) : R4::zero();
                pm[j] = !valid ? 0 : mask ? (int)mask[tok0 + t0 + tp] : 1;   // raw mask byte
            }
        }
        {
            // v or d_o, this workgroup's columns
            const int tp = tid / 16;
            const bool valid = tp < nt;
            py = valid ? ld4(y_src + cb, (unsigned)(tp * H * D + kChainCols * cg + 4 * (tid % 16))) : R4::zero();
            pmy = !valid ? 0 : (GDN || !mask) ? 1 : (int)mask[tok0 + t0 + tp];
        }
    };
    // With one staging unit per thread the next chunk's inputs are loaded
    // while the current one is processed; with two (D = 128) the other
    // workgroups on the CU cover the load latency instead.
    constexpr bool kAhead = NU == 1;
    if (kAhead && nck > 0) fetch(fwd ? 0 : nck - 1, tid0);
    for (int it = 0; it < nck; ++it) {
        // The lane indices pass through an empty asm here, so that values
        // derived from them (addresses, masks, constants) are formed inside
        // the loop instead of being hoisted and held in registers next to
        // the state across every chunk.
        int tid = tid0, q = q0, m = m0;
        asm volatile("" : "+v"(tid), "+v"(q), "+v"(m));
        const int lane = 16 * q + m;
        const int c = fwd ? it : nck - 1 - it;
        const int Lc = min(kL, T - c * kL);
        if (!kAhead) fetch(c, tid);
        if (c < nck_store) store_slice<D>((fwd ? ckpt : dck) + ckidx(c) * D * D, St, q, cw + m);
        __syncthreads();   // every wave is done with the previous chunk's tiles
        // the mask bytes enter the comparisons only here (an empty asm keeps
        // the compiler from comparing them right after their loads, which
        // would make the wave wait for every load and store in flight)
        asm volatile("" : "+v"(pmy));
#pragma unroll
        for (int j = 0; j < NU; ++j) asm volatile("" : "+v"(pm[j]));
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int tp = tpj(tid, j), cp = cpj(tid, j);
            if constexpr (GDN) {
                const f32x4 k4 = R4::f32(pf[j][0]);
                const f32x4 kn = k4 * inv_norm<D>(k4);
                const f32x4 q4 = R4::f32(pf[j][1]);
                const float iq = inv_norm<D>(q4);   // unused in the forward role (q4 = 0 there)
                const float gg = pg[j], bt = pb[j];
                *(f32x4 *)&s.G[tp][cp] = f32x4{gg, gg, gg, gg};
                *(f32x4 *)&s.A[tp][cp] = kn * (-__expf(gg) * bt);
                *(f32x4 *)&s.B[tp][cp] = kn;
                *(f32x4 *)&s.X[tp][cp] = fwd ? kn * bt : q4 * iq;
            } else {
                // a token that does not update gets w = a = b = 0 (an identity
                // step) and, in the forward role, k = v = 0; the backward role
                // keeps r and d_o (a masked token still reads the state)
                const bool up = pm[j] != 0;
                *(f32x4 *)&s.G[tp][cp] = up ? R4::f32(pf[j][0]) : z;
                *(f32x4 *)&s.A[tp][cp] = up ? R4::f32(pf[j][1]) : z;
                *(f32x4 *)&s.B[tp][cp] = up ? R4::f32(pf[j][2]) : z;
                *(f32x4 *)&s.X[tp][cp] = (up || !fwd) ? R4::f32(pf[j][3]) : z;
            }
            if (cp == 0) s.upd[tp] = pm[j] != 0;
        }
        *(typename R4::type *)&s.Y[tid / 16][4 * (tid % 16)] = (pmy != 0 || !fwd) ? py : R4::zero();
        __syncthreads();
        if (kAhead && it + 1 < nck) fetch(fwd ? c + 1 : c - 1, tid);
        int extreme = 0;
        if (tid < D) {
            float x[kL];
#pragma unroll
            for (int t = 0; t < kL; ++t) x[t] = s.G[t][tid];
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < kL; ++t) {
                extreme |= x[t] > 0.0f;
                acc += x[t];
                s.G[t][tid] = acc;
            }
            extreme |= acc < kMinChunkLogDecay;
            s.EGL[tid] = __expf(acc);
        }
        const int cl = 16 * wave + m;   // this lane's column in the value tile
        if (__syncthreads_or(extreme)) {
            // token by token on the raw operands, with raw w read again into
            // G (the prefix replaced it); tokens that do not update get w = 0
            {
                const size_t t0 = (size_t)c * kL;
#pragma unroll
                for (int j = 0; j < NU; ++j) {
                    const int tp = tpj(tid, j), cp = cpj(tid, j);
                    const bool up = s.upd[tp] != 0;
                    if constexpr (GDN) {
                        const float gg = up ? ld1(w + (tok0 + t0) * H + h, (unsigned)(tp * H)) : 0.0f;
                        *(f32x4 *)&s.G[tp][cp] = f32x4{gg, gg, gg, gg};
                    } else {
                        *(f32x4 *)&s.G[tp][cp] =
                            up ? R4::f32(ld4(w + ((tok0 + t0) * H + h) * D, (unsigned)(tp * H * D + cp))) : z;
                    }
                }
            }
            __syncthreads();
            const auto &W = s.G;
            if (fwd) {
                for (int t = 0; t < Lc; ++t) {
                    if (!s.upd[t]) continue;
                    float sb = 0.0f;
#pragma unroll
                    for (int ti = 0; ti < NTILE; ++ti) {
                        const f32x4 bt = *(const f32x4 *)&s.B[t][16 * ti + 4 * q];
#pragma unroll
                        for (int i = 0; i < 4; ++i) sb = fmaf(bt[i], St[ti][i], sb);
                    }
                    sb = xsum32(xsum16(sb));
                    const float vj = tl(s.Y[t][cl]);
#pragma unroll
                    for (int ti = 0; ti < NTILE; ++ti) {
                        const int r0 = 16 * ti + 4 * q;
                        const f32x4 wt = *(const f32x4 *)&W[t][r0], at = *(const f32x4 *)&s.A[t][r0];
                        const f32x4 xt = *(const f32x4 *)&s.X[t][r0];
#pragma unroll
                        for (int i = 0; i < 4; ++i) St[ti][i] = fmaf(__expf(wt[i]), St[ti][i], fmaf(at[i], sb, xt[i] * vj));
                    }
                }
            } else {
                for (int t = Lc - 1; t >= 0; --t) {
                    const float doj = tl(s.Y[t][cl]);
                    float ad = 0.0f;
#pragma unroll
                    for (int ti = 0; ti < NTILE; ++ti) {
                        const int r0 = 16 * ti + 4 * q;
                        const f32x4 xt = *(const f32x4 *)&s.X[t][r0], at = *(const f32x4 *)&s.A[t][r0];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            St[ti][i] = fmaf(xt[i], doj, St[ti][i]);
                            ad = fmaf(at[i], St[ti][i], ad);
                        }
                    }
                    if (!s.upd[t]) continue;
                    ad = xsum32(xsum16(ad));
#pragma unroll
                    for (int ti = 0; ti < NTILE; ++ti) {
                        const int r0 = 16 * ti + 4 * q;
                        const f32x4 wt = *(const f32x4 *)&W[t][r0], bt = *(const f32x4 *)&s.B[t][r0];
#pragma unroll
                        for (int i = 0; i < 4; ++i) St[ti][i] = fmaf(__expf(wt[i]), St[ti][i], bt[i] * ad);
                    }
                }
            }
            continue;
        }
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int tp = tpj(tid, j), cp = cpj(tid, j);
            const f32x4 G = *(const f32x4 *)&s.G[tp][cp];
            const f32x4 Gp = tp ? *(const f32x4 *)&s.G[tp - 1][cp] : z;
            f32x4 eG, enG, eGp;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                eG[i] = __expf(G[i]);
                enG[i] = __expf(-G[i]);
                eGp[i] = __expf(Gp[i]);
            }
            *(f32x4 *)&s.A[tp][cp] *= enG;
            *(f32x4 *)&s.B[tp][cp] *= eGp;
            *(f32x4 *)&s.X[tp][cp] *= fwd ? enG : eG;
        }
        __syncthreads();   // G is dead from here: M and T take its place
        // Chunk matrices, each wave one of the two over one half of the
        // channels: mi = wave & 1 (M_ba; M_bk forward, M_ra backward), half
        // wave >> 1.  M_ba and M_bk are strictly lower, M_ra keeps the
        // diagonal; M_ba is stored in both orientations.
        {
            const int mi = wave & 1, hf = wave >> 1;
            const float(*P)[Lds::LD] = (mi == 0 || fwd) ? s.B : s.X;
            const float(*Q)[Lds::LD] = (mi == 1 && fwd) ? s.X : s.A;
            f32x4 acc = z;
#pragma unroll
            for (int j0b = 0; j0b < D / 2; j0b += 16) {
                const int j = hf * (D / 2) + j0b + 4 * q;
                const f32x4 xa = *(const f32x4 *)&P[m][j], yb = *(const f32x4 *)&Q[m][j];
#pragma unroll
                for (int st = 0; st < 4; ++st) acc = mfma_f32(xa[st], yb[st], acc);
            }
            const bool strict = mi == 0 || fwd;
            f32x4 keep;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * q + i;
                keep[i] = (strict ? row > m : row >= m) ? acc[i] : 0.0f;
            }
            float(*Mw)[20] = s.M[mi == 0 ? hf : 4 + hf];
#pragma unroll
            for (int i = 0; i < 4; ++i) Mw[4 * q + i][m] = keep[i];
            if (mi == 0) *(f32x4 *)&s.M[2 + hf][m][4 * q] = keep;
        }
        __syncthreads();
        // T = (I - M_ba)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8) with
        // N = M_ba strictly lower (N^16 = 0), formed by wave 0 on the matrix
        // cores and handed to the other waves through LDS (each wave forming
        // it itself loads the matrix cores with four times the products).
        // acc(X) is the accumulator layout of X (lane (q, m) holds rows
        // 4q .. 4q + 3 of column m); with the contraction index permuted as
        // elsewhere, acc(X Y) = sum_st mfma(acc(X^T)[st], acc(Y)[st]), so each
        // product needs its left factor transposed.  The forward role reads
        // rows of T (U = T X): acc(T^T); the backward role reads columns
        // (dX = T^T dU): acc(T).  Every lane (q, m) ends with tq =
        // T[m][4q + i] (forward) or T[4q + i][m] (backward).
        f32x4 tq;
        if (wave == 0) {
            auto mm = [](f32x4 aT, f32x4 b) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) c = mfma_f32(aT[st], b[st], c);
                return c;
            };
            const f32x4 nA = *(const f32x4 *)&s.M[2][m][4 * q] + *(const f32x4 *)&s.M[3][m][4 * q];   // acc(N)
            const f32x4 nT = *(const f32x4 *)&s.M[0][m][4 * q] + *(const f32x4 *)&s.M[1][m][4 * q];   // acc(N^T)
            f32x4 eye;
#pragma unroll
            for (int i = 0; i < 4; ++i) eye[i] = 4 * q + i == m ? 1.0f : 0.0f;
            const f32x4 n2 = mm(nT, nA), n2T = mm(nA, nT);
            const f32x4 n4 = mm(n2T, n2), n4T = mm(n2, n2T);
            const f32x4 n8 = mm(n4T, n4);
            const f32x4 p1T = mm(eye + n2, eye + nT);   // ((I + N)(I + N^2))^T
            const f32x4 p2T = mm(eye + n4, p1T);        // (P1 (I + N^4))^T
            // each lane's tq, over the transposed M_ba slot that only this wave reads
            *(f32x4 *)&s.M[2][m][4 * q] = fwd ? mm(eye + n8, p2T) : mm(p2T, eye + n8);
        }
        __syncthreads();
        tq = *(const f32x4 *)&s.M[2][m][4 * q];
        // M_bk (forward) or M_ra (backward), the sum of its two halves
        auto m2 = [&](int r, int c2) { return s.M[4][r][c2] + s.M[5][r][c2]; };
        const int c0 = 16 * wave;   // this wave's columns in the value tile
        if (fwd) {
            // X = B~ S + M_bk V
            f32x4 Xa = z;
#pragma unroll
            for (int ti = 0; ti < NTILE; ++ti) {
                const f32x4 bt = *(const f32x4 *)&s.B[m][16 * ti + 4 * q];
#pragma unroll
                for (int i = 0; i < 4; ++i) Xa = mfma_f32(bt[i], St[ti][i], Xa);
            }
            Xa = mm16<kL>(Xa, [&](int mm, int kk) { return m2(mm, kk); },
                          [&](int kk, int n) { return tl(s.Y[kk][c0 + n]); }, lane);
            // U = T X (X's token rows 4q + i are this lane's; tq = T[m][4q + i])
            f32x4 U = z;
#pragma unroll
            for (int i = 0; i < 4; ++i) U = mfma_f32(tq[i], Xa[i], U);
            // S <- diag(e^{G_L}) (S + A^T U + K^T V)
            float vy[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) vy[i] = tl(s.Y[4 * q + i][c0 + m]);
#pragma unroll
            for (int ti = 0; ti < NTILE; ++ti) {
                f32x4 acc = St[ti];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = mfma_f32(s.A[4 * q + i][16 * ti + m], U[i], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = mfma_f32(s.X[4 * q + i][16 * ti + m], vy[i], acc);
                St[ti] = acc * *(const f32x4 *)&s.EGL[16 * ti + 4 * q];
            }
        } else {
            // dY = diag(e^{G_L}) dS', formed tile by tile where it is used
            auto dY = [&](int ti) { return St[ti] * *(const f32x4 *)&s.EGL[16 * ti + 4 * q]; };
            // dU = A^ dY + M_ra^T dO
            f32x4 dU = z;
#pragma unroll
            for (int ti = 0; ti < NTILE; ++ti) {
                const f32x4 at = *(const f32x4 *)&s.A[m][16 * ti + 4 * q];
                const f32x4 y = dY(ti);
#pragma unroll
                for (int i = 0; i < 4; ++i) dU = mfma_f32(at[i], y[i], dU);
            }
            dU = mm16<kL>(dU, [&](int mm, int kk) { return m2(kk, mm); },
                          [&](int kk, int n) { return tl(s.Y[kk][c0 + n]); }, lane);
            // dX = T^T dU (tq = T[4q + i][m])
            f32x4 dX = z;
#pragma unroll
            for (int i = 0; i < 4; ++i) dX = mfma_f32(tq[i], dU[i], dX);
            // dS <- dY + R~^T dO + B~^T dX
            float oy[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) oy[i] = tl(s.Y[4 * q + i][c0 + m]);
#pragma unroll
            for (int ti = 0; ti < NTILE; ++ti) {
                f32x4 acc = dY(ti);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = mfma_f32(s.X[4 * q + i][16 * ti + m], oy[i], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = mfma_f32(s.B[4 * q + i][16 * ti + m], dX[i], acc);
                St[ti] = acc;
            }
        }
    }
    if (!fwd && d_s0) store_slice<D>(d_s0 + st, St, q0, cw + m0);
}

// ck_off[0..nseq]: exclusive prefix sums of the sequences' chunk counts
// (offsets clamped as in seq_range), saturating at cap.  One workgroup
// scanning 256 sequences at a time.
__global__ __launch_bounds__(256) void chunk_offsets_kernel(const int32_t *__restrict__ cu, int nseq, int total_T,
                                                            long long cap, int32_t *__restrict__ ck_off)
{
    __shared__ long long part[256];
    long long carry = 0;
    SeqGeom vg;
    vg.cu = cu;
    vg.total_T = total_T;
    for (int base = 0; base < nseq; base += 256) {
        const int n = base + (int)threadIdx.x;
        long long cnt = 0;
        if (n < nseq) {
            int tb, te;
            seq_range(vg, n, tb, te);
            cnt = (te - tb + kL - 1) / kL;
        }
        part[threadIdx.x] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const long long add = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
            __syncthreads();
            part[threadIdx.x] += add;
            __syncthreads();
        }
        if (n < nseq) ck_off[n + 1] = (int32_t)min(carry + part[threadIdx.x], cap);
        carry += part[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) ck_off[0] = 0;
}

template <int D, typename T_IO, bool GDN>
hipError_t launch_bwd_d(const BwdArgs &p, hipStream_t stream)
{
    const size_t nbh = (size_t)p.B * p.H;
    SeqGeom vg;
    size_t nck, grid2;
    if (p.cu_seqlens) {
        // packed: checkpoints [capacity][H], then the chunk offsets
        const long long cap = bwd_varlen_chunk_capacity(p.B, p.T);
        nck = (size_t)cap;
        int32_t *ck_off = (int32_t *)((char *)p.ws + sizeof(float) * (size_t)cap * p.H * D * D * 2);
        hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(256), 0, stream, p.cu_seqlens, p.B, p.T, cap, ck_off);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        vg.cu = p.cu_seqlens;
        vg.ck_off = ck_off;
        vg.smap = p.state_map;
        vg.n_state = p.n_state;
        vg.nseq = p.B;
        vg.total_T = p.T;
        grid2 = (size_t)cap * p.H;
    } else {
        nck = (size_t)(p.T + kL - 1) / kL;
        grid2 = nbh * nck;
        vg.n_state = p.n_state;
    }
    float *ckpt = (float *)p.ws;
    float *dck = ckpt + (p.cu_seqlens ? nck * p.H : nbh * nck) * D * D;
    // (role, sequence-head) pairs in blocks of eight, each block once per column group
    const size_t grid1 = (2 * nbh + 7) / 8 * 8 * (D / kChainCols);
    // packed calls of few sequences run the recurrences longest first
    auto chain = use_longest_first(p.cu_seqlens != nullptr, p.B, p.T) ? chain_kernel<D, T_IO, GDN, true>
                                                            : chain_kernel<D, T_IO, GDN, false>;
    hipLaunchKernelGGL(chain, dim3((unsigned)grid1), dim3(kChainWaves * kWave), 0, stream, p.T,
                       p.H, (int)nbh, (const T_IO *)p.r, (const T_IO *)p.w, (const T_IO *)p.k,
                       (const T_IO *)p.v, (const T_IO *)p.a, (const T_IO *)p.b, p.s0, p.mask,
                       (const T_IO *)p.d_o, p.d_sf, ckpt, dck, p.d_s0, vg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (grid2 == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_grad_kernel<D, T_IO, GDN>), dim3((unsigned)grid2), dim3(D * 4), 0, stream, p.T,
                       p.H, (int)nck, (const T_IO *)p.r, (const T_IO *)p.w, (const T_IO *)p.k, (const T_IO *)p.v,
                       (const T_IO *)p.a, (const T_IO *)p.b, p.mask, (const T_IO *)p.d_o, ckpt, dck,
                       (T_IO *)p.dr, (T_IO *)p.dw, (T_IO *)p.dk, (T_IO *)p.dv, (T_IO *)p.da, (T_IO *)p.db, vg);
    return hipGetLastError();
}

}  // namespace

size_t bwd_checkpoint_bytes(int B, int T, int H, int D)
{
    const size_t nck = ((size_t)T + kL - 1) / kL;
    return sizeof(float) * (size_t)B * H * D * D * 2 * nck;
}

size_t bwd_workspace_bytes(int B, int T, int H, int D)
{
    // checkpoints, then per-sequence initial-state gradients (summed into
    // the gradient of a shared initial state), 256-byte aligned
    const size_t ck = (bwd_checkpoint_bytes(B, T, H, D) + 255) / 256 * 256;
    return ck + sizeof(float) * (size_t)B * H * D * D;
}

long long bwd_varlen_chunk_capacity(int B, int T)
{
    return ((long long)T + kL - 1) / kL + B;
}

size_t bwd_varlen_workspace_bytes(int B, int T, int H, int D)
{
    const size_t cap = (size_t)bwd_varlen_chunk_capacity(B, T);
    return sizeof(float) * cap * H * D * D * 2 + sizeof(int32_t) * ((size_t)B + 1);
}

template <bool GDN>
hipError_t launch_bwd_g(int dtype, const BwdArgs &p, hipStream_t stream)
{
    if (p.D == 64)
        return dtype == 0 ? launch_bwd_d<64, float, GDN>(p, stream) : launch_bwd_d<64, uint16_t, GDN>(p, stream);
    return dtype == 0 ? launch_bwd_d<128, float, GDN>(p, stream) : launch_bwd_d<128, uint16_t, GDN>(p, stream);
}

hipError_t launch_backward(int dtype, const BwdArgs &p, hipStream_t stream)
{
    return p.gdn ? launch_bwd_g<true>(dtype, p, stream) : launch_bwd_g<false>(dtype, p, stream);
}

}  // namespace wkv7

// Chunked WKV7 forward on bf16 MFMA (bf16 I/O, fp32 state).
//
// The recurrence (rwkv-ops README, section "rwkv7op 使用方法", read as the
// generalized delta rule) is evaluated 16 tokens at a time.  Within a chunk
// with start state S (K x V, fp32), log-decay prefix G_i = sum_{m<=i} w_m and
// G_{-1} = 0 (per channel), u_i = b_i^T S_{i-1} unrolls to
//
//   U   = T (B~ S + M_bk V)                    T = (I - M_ba)^-1
//   O   = R~ S + M_ra U + M_rk V
//   S' = diag(e^{G_L}) S + A~^T U + K~^T V
//
// with  R~ = r e^{G},  B~ = b e^{G_{i-1}},  A^ = a e^{-G},  K^ = k e^{-G},
// A~ = a e^{G_L - G},  K~ = k e^{G_L - G},  M_ba = B~ A^^T and M_bk = B~ K^^T
// strictly lower, M_ra = R~ A^^T and M_rk = R~ K^^T lower with diagonal.
// Every factor of the form e^{G_i - G_j} with j <= i is <= 1, and the split
// factors stay finite while the chunk's decay sum is above -60; chunks beyond
// that (or with w > 0) take an exact token-by-token path instead.  A token
// with mask 0 (or past T) gets w = a = k = 0, an exact identity step.
//
// Layout of the work.  One workgroup per (b, h) holds the state in MFMA
// accumulator layout: wave w owns columns [16w, 16w+16), lane (g = l/16,
// j = l%16) rows 16q + 4g + i of column 16w + j.  Each super-step handles NP
// chunks: first wave p < NP prepares chunk c0 + p on its own (no cross-wave
// traffic) and leaves every operand of the serial step in its LDS slot, in
// per-lane fragment order; after a barrier all waves run the short S-dependent
// chain for the NP chunks on their columns.  The raw tiles of the next
// super-step are requested before the serial phase so their latency hides
// behind it.
//
// Precision.  MFMA operands are bf16 with fp32 accumulation; the r.k and b.k
// chunk matrices use a hi/lo split (3 products) and every product with the
// exact-bf16 value tile V splits its left operand (2 products), which keeps the
// error near the bf16 rounding of the output.
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace wkv7 {

// A chunk whose summed decay factor exp(G_L) falls below e^-60 in any channel
// would need factors up to e^60 in the split form; it takes the exact path.
constexpr float kMinChunkFactor = 8.75651076e-27f;   // e^-60

template <int D> struct CK {
    static constexpr int NW = D / 16;              // waves = 16-column state slices
    static constexpr int NT = NW * kWave;
    static constexpr int NP = (D == 64) ? 4 : 2;   // chunks per super-step
    static constexpr int NCB = D / 32;             // 32-channel blocks
    static constexpr int NRT = D / 16;             // 16-row state tiles
    // Slot layout in bytes; fragments are 64 lanes x (16 or 8) bytes.
    static constexpr int OFF_B = 0;                       // B~ A-frags, NCB x 1024
    static constexpr int OFF_R = OFF_B + NCB * 1024;      // R~ A-frags
    static constexpr int OFF_TINV = OFF_R + NCB * 1024;   // T A-frag (16x16x16)
    static constexpr int OFF_NBKH = OFF_TINV + 512;
    static constexpr int OFF_NBKL = OFF_NBKH + 512;
    static constexpr int OFF_MRA = OFF_NBKL + 512;
    static constexpr int OFF_MRKH = OFF_MRA + 512;
    static constexpr int OFF_MRKL = OFF_MRKH + 512;
    static constexpr int OFF_AT = OFF_MRKL + 512;         // A~^T A-frags, NRT x 512
    static constexpr int OFF_KTH = OFF_AT + NRT * 512;
    static constexpr int OFF_KTL = OFF_KTH + NRT * 512;
    static constexpr int OFF_V = OFF_KTL + NRT * 512;     // V B-frags per 16 columns
    static constexpr int OFF_EGL = OFF_V + NW * 512;      // e^{G_L}, D floats
    static constexpr int OFF_FLAG = OFF_EGL + D * 4;
    static constexpr int SLOT = OFF_FLAG + 16;
    static constexpr int LDS = NP * SLOT;
};

// Raw bf16 tiles of one chunk in the precompute lane layout: lane (t = l%16,
// g = l/16) holds token t, channels 32s + 4g + {0..3} (x[s][*][0]) and
// 32s + 16 + 4g + {0..3} (x[s][*][1]).  Array order: r, w, k, a, b, v.
template <int D> struct RawTile {
    u32x2 x[CK<D>::NCB][6][2];
    int upd;     // token updates the state
    int valid;   // token exists (t0 + t < T)
};

template <int D>
__device__ __forceinline__ void load_raw(RawTile<D> &rt, const uint16_t *const *src,
                                         const uint8_t *mask, int T, int H, int bb, int h,
                                         int chunk, int lane)
{
    const int t = lane & 15, g = lane >> 4;
    const int tok = chunk * 16 + t;
    rt.valid = tok < T;
    rt.upd = rt.valid && (mask == nullptr || mask[(size_t)bb * T + tok] != 0);
    const size_t base = (((size_t)bb * T + (rt.valid ? tok : 0)) * H + h) * D + 4 * g;
    // Unconditional loads (tokens past T read token 0 of the sequence); the
    // values of tokens that do not update are zeroed where they are used.
#pragma unroll
    for (int arr = 0; arr < 6; ++arr) {
        const u32x2 *p = (const u32x2 *)(src[arr] + base);   // 8-byte units
#pragma unroll
        for (int s = 0; s < CK<D>::NCB; ++s)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) rt.x[s][arr][hh] = p[8 * s + 4 * hh];
    }
}

// Make a token that does not update an exact identity step: w, k, a, b (and
// v when staged) are cleared, so that whatever they hold (even inf or nan)
// cannot reach the state; r stays, since such a token still emits an
// output.  A token past T is inert (r = 0 as well).
template <int D>
__device__ __forceinline__ void zero_inactive(RawTile<D> &rt, int narr)
{
    if (__all(rt.upd)) return;
#pragma unroll
    for (int s = 0; s < CK<D>::NCB; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int arr = 1; arr <= 4; ++arr)
                rt.x[s][arr][hh] = rt.upd ? rt.x[s][arr][hh] : u32x2{0u, 0u};
            rt.x[s][0][hh] = rt.valid ? rt.x[s][0][hh] : u32x2{0u, 0u};
            if (narr > 5) rt.x[s][5][hh] = rt.upd ? rt.x[s][5][hh] : u32x2{0u, 0u};
        }
}

__device__ __forceinline__ void unpack8(const u32x2 *x, float *out)
{
    out[0] = bf16_lo(x[0][0]); out[1] = bf16_hi(x[0][0]);
    out[2] = bf16_lo(x[0][1]); out[3] = bf16_hi(x[0][1]);
    out[4] = bf16_lo(x[1][0]); out[5] = bf16_hi(x[1][0]);
    out[6] = bf16_lo(x[1][1]); out[7] = bf16_hi(x[1][1]);
}

__device__ __forceinline__ bf16x8 pack8(const float *x)
{
    const u32x4 p = {cvt2_bits(x[0], x[1]), cvt2_bits(x[2], x[3]), cvt2_bits(x[4], x[5]),
                     cvt2_bits(x[6], x[7])};
    return __builtin_bit_cast(bf16x8, p);
}

// hi/lo split: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo)
{
    hi = pack8(x);
    float rem[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rem[e] = x[e] - (float)hi[e];
    lo = pack8(rem);
}

__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo)
{
    hi = cvt4(x);
    f32x4 rem;
#pragma unroll
    for (int i = 0; i < 4; ++i) rem[i] = x[i] - (float)hi[i];
    lo = cvt4(rem);
}

__device__ __forceinline__ void st8(char *p, bf16x4 v) { *(bf16x4 *)p = v; }
__device__ __forceinline__ void st16(char *p, bf16x8 v) { *(bf16x8 *)p = v; }
__device__ __forceinline__ bf16x4 ld8(const char *p) { return *(const bf16x4 *)p; }
__device__ __forceinline__ bf16x8 ld16(const char *p) { return *(const bf16x8 *)p; }

// Prepare every S-independent operand of one chunk into its LDS slot.
// Executed by one wave; `psel[hh]` is the B-fragment that copies channel half
// hh of a 32-channel block to a token-contiguous (transposed) accumulator.
template <int D>
__device__ void precompute(RawTile<D> rt, char *slot, int lane, const bf16x8 *psel)
{
    using C = CK<D>;
    const int t = lane & 15, g = lane >> 4;
    (void)t;
    f32x4 mraT = zero4(), mrkT = zero4(), mba = zero4(), mbaT = zero4(), mbk = zero4();
    bool extreme = false;
    zero_inactive<D>(rt, 6);

#pragma unroll
    for (int s = 0; s < C::NCB; ++s) {
        float rv[8], wv[8], kv[8], av[8], bv[8];
        unpack8(rt.x[s][0], rv);
        unpack8(rt.x[s][1], wv);
        unpack8(rt.x[s][2], kv);
        unpack8(rt.x[s][3], av);
        unpack8(rt.x[s][4], bv);
        float Rt[8], Bt[8], Ah[8], Kh[8], At[8], Kt[8];
        int wmax = (int)0x80000000;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // Positive w (as signed integer bits: > 0) leaves the fast path.
            wmax = max(wmax, __float_as_int(wv[e]));
            // Prefix in log2 units: e^{G} = 2^{G2}.
            const float G2 = row_scan16(wv[e] * 1.4426950408889634f);
            const float eG = __builtin_amdgcn_exp2f(G2);
            const float enG = __builtin_amdgcn_exp2f(-G2);
            const float eGp = row_shr<1>(eG, 1.0f);
            const float eGL = row_bcast15(eG);
            extreme |= eGL < kMinChunkFactor;
            Rt[e] = rv[e] * eG;
            Bt[e] = bv[e] * eGp;
            Ah[e] = av[e] * enG;
            Kh[e] = kv[e] * enG;
            At[e] = Ah[e] * eGL;
            Kt[e] = Kh[e] * eGL;
            if (t == 0) {
                const int ch = 32 * s + 4 * g + (e & 3) + 16 * (e >> 2);
                *(float *)(slot + C::OFF_EGL + ch * 4) = eGL;
            }
        }
        extreme |= wmax > 0;
        bf16x8 Rh, Rl, Bh, Bl, Khh, Khl, Kth, Ktl;
        split8(Rt, Rh, Rl);
        split8(Bt, Bh, Bl);
        split8(Kh, Khh, Khl);
        split8(Kt, Kth, Ktl);
        const bf16x8 Ahh = pack8(Ah);
        const bf16x8 Ath = pack8(At);
        // v already holds bf16 values: reinterpret the raw bits.
        const u32x4 vbits = {rt.x[s][5][0][0], rt.x[s][5][0][1], rt.x[s][5][1][0], rt.x[s][5][1][1]};
        const bf16x8 Vb = __builtin_bit_cast(bf16x8, vbits);

        // Chunk matrices, contraction over this block's 32 channels.
        mraT = mfma32(Ahh, Rh, mraT);                 // (R~ A^^T)^T
        mrkT = mfma32(Khh, Rh, mrkT);                 // (R~ K^^T)^T, hi/lo split
        mrkT = mfma32(Khl, Rh, mrkT);
        mrkT = mfma32(Khh, Rl, mrkT);
        mba = mfma32(Bh, Ahh, mba);                   // B~ A^^T
        mbaT = mfma32(Ahh, Bh, mbaT);                 // (B~ A^^T)^T
        mbk = mfma32(Bh, Khh, mbk);                   // B~ K^^T, hi/lo split
        mbk = mfma32(Bh, Khl, mbk);
        mbk = mfma32(Bl, Khh, mbk);

        // Operands contracted over channels with the state: fragment order.
        st16(slot + C::OFF_B + s * 1024 + lane * 16, Bh);
        st16(slot + C::OFF_R + s * 1024 + lane * 16, Rh);

        // Operands contracted over tokens: transpose with a selection MFMA
        // (exact: bf16 values times 1.0 accumulated in fp32).
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int q = 2 * s + hh;
            st8(slot + C::OFF_AT + q * 512 + lane * 8, cvt4(mfma32(Ath, psel[hh], zero4())));
            st8(slot + C::OFF_KTH + q * 512 + lane * 8, cvt4(mfma32(Kth, psel[hh], zero4())));
            st8(slot + C::OFF_KTL + q * 512 + lane * 8, cvt4(mfma32(Ktl, psel[hh], zero4())));
            st8(slot + C::OFF_V + q * 512 + lane * 8, cvt4(mfma32(Vb, psel[hh], zero4())));
        }
    }

    // Causal masks in accumulator layout: element (row = 4g + i, col = j).
    const int j = lane & 15;
    f32x4 eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        mba[i] = row > j ? mba[i] : 0.0f;       // M_ba strictly lower
        mbk[i] = row > j ? mbk[i] : 0.0f;       // M_bk strictly lower
        mbaT[i] = j > row ? mbaT[i] : 0.0f;     // transpose of strictly lower
        mraT[i] = j >= row ? mraT[i] : 0.0f;    // transpose of lower with diagonal
        mrkT[i] = j >= row ? mrkT[i] : 0.0f;
        eye[i] = row == j ? 1.0f : 0.0f;
    }

    // T = (I - M_ba)^-1 = (I + N^8)(I + N^4)(I + N^2)(I + N), N = M_ba
    // nilpotent.  Each matrix X is carried as acc(X) and acc(X^T); then
    // acc(XY) = mfma(acc(X^T), acc(Y)) and acc((XY)^T) = mfma(acc(Y), acc(X^T)).
    const bf16x4 n1 = cvt4(mba), n1t = cvt4(mbaT);
    const f32x4 p2 = mfma16(n1t, n1, zero4()), p2t = mfma16(n1, n1t, zero4());
    const bf16x4 n2 = cvt4(p2), n2t = cvt4(p2t);
    const f32x4 p4 = mfma16(n2t, n2, zero4()), p4t = mfma16(n2, n2t, zero4());
    const bf16x4 n4 = cvt4(p4), n4t = cvt4(p4t);
    const bf16x4 n8t = cvt4(mfma16(n4, n4t, zero4()));
    const f32x4 t1 = eye + mba, t1t = eye + mbaT;
    const bf16x4 t1b = cvt4(t1);
    const f32x4 t2 = mfma16(n2t, t1b, t1), t2t = mfma16(t1b, n2t, t1t);
    const bf16x4 t2b = cvt4(t2);
    const f32x4 t4 = mfma16(n4t, t2b, t2), t4t = mfma16(t2b, n4t, t2t);
    const f32x4 t8t = mfma16(cvt4(t4), n8t, t4t);        // acc(T^T) = A-frag of T
    const bf16x4 tinv = cvt4(t8t);
    st8(slot + C::OFF_TINV + lane * 8, tinv);

    // N_bk = T M_bk, stored as A-frag: acc(N_bk^T) = mfma(acc(M_bk), acc(T^T)).
    bf16x4 hi, lo;
    split4(mfma16(cvt4(mbk), tinv, zero4()), hi, lo);
    st8(slot + C::OFF_NBKH + lane * 8, hi);
    st8(slot + C::OFF_NBKL + lane * 8, lo);
    st8(slot + C::OFF_MRA + lane * 8, cvt4(mraT));
    split4(mrkT, hi, lo);
    st8(slot + C::OFF_MRKH + lane * 8, hi);
    st8(slot + C::OFF_MRKL + lane * 8, lo);

    const int any_extreme = __any((int)extreme);
    if (lane == 0) *(int *)(slot + C::OFF_FLAG) = any_extreme;
}

// Exact fp32 token-by-token update of this wave's 16 columns for one chunk.
template <int D>
__device__ void chunk_exact(f32x4 *S, const uint16_t *r, const uint16_t *w, const uint16_t *k,
                            const uint16_t *v, const uint16_t *a, const uint16_t *b,
                            const uint8_t *mask, uint16_t *o, int T, int H, int bb, int h,
                            int chunk, int wave, int lane)
{
    const int g = lane >> 4, j = lane & 15;
    const int col = wave * 16 + j;
    for (int tt = 0; tt < 16; ++tt) {
        const int tok = chunk * 16 + tt;
        if (tok >= T) break;
        const bool upd = mask == nullptr || mask[(size_t)bb * T + tok] != 0;
        const size_t base = (((size_t)bb * T + tok) * H + h) * D;
        if (upd) {
            float sb = 0.0f;
#pragma unroll
            for (int q = 0; q < D / 16; ++q) {
                const u32x2 bq = *(const u32x2 *)(b + base + 16 * q + 4 * g);
                sb += bf16_lo(bq[0]) * S[q][0] + bf16_hi(bq[0]) * S[q][1] +
                      bf16_lo(bq[1]) * S[q][2] + bf16_hi(bq[1]) * S[q][3];
            }
            sb = xor_sum(sb, 16);
            sb = xor_sum(sb, 32);
            const float vj = bf16_bits_to_f32(v[base + col]);
#pragma unroll
            for (int q = 0; q < D / 16; ++q) {
                const u32x2 wq = *(const u32x2 *)(w + base + 16 * q + 4 * g);
                const u32x2 aq = *(const u32x2 *)(a + base + 16 * q + 4 * g);
                const u32x2 kq = *(const u32x2 *)(k + base + 16 * q + 4 * g);
                const float we[4] = {bf16_lo(wq[0]), bf16_hi(wq[0]), bf16_lo(wq[1]), bf16_hi(wq[1])};
                const float ae[4] = {bf16_lo(aq[0]), bf16_hi(aq[0]), bf16_lo(aq[1]), bf16_hi(aq[1])};
                const float ke[4] = {bf16_lo(kq[0]), bf16_hi(kq[0]), bf16_lo(kq[1]), bf16_hi(kq[1])};
#pragma unroll
                for (int i = 0; i < 4; ++i) S[q][i] = fmaf(__expf(we[i]), S[q][i], fmaf(ae[i], sb, ke[i] * vj));
            }
        }
        float ov = 0.0f;
#pragma unroll
        for (int q = 0; q < D / 16; ++q) {
            const u32x2 rq = *(const u32x2 *)(r + base + 16 * q + 4 * g);
            ov += bf16_lo(rq[0]) * S[q][0] + bf16_hi(rq[0]) * S[q][1] +
                  bf16_lo(rq[1]) * S[q][2] + bf16_hi(rq[1]) * S[q][3];
        }
        ov = xor_sum(ov, 16);
        ov = xor_sum(ov, 32);
        if (g == 0) o[base + col] = f32_to_bf16_bits(ov);
    }
}

// The S-dependent part of one chunk for this wave's 16 columns.
template <int D>
__device__ __forceinline__ void chunk_serial(f32x4 *S, const char *slot, uint16_t *o, int T, int H,
                                             int bb, int h, int chunk, int wave, int lane)
{
    using C = CK<D>;
    const int g = lane >> 4, j = lane & 15;
    f32x4 X = zero4(), O = zero4();
#pragma unroll
    for (int s = 0; s < C::NCB; ++s) {
        const bf16x4 lo4 = cvt4(S[2 * s]), hi4 = cvt4(S[2 * s + 1]);
        const bf16x8 sb = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        X = mfma32(ld16(slot + C::OFF_B + s * 1024 + lane * 16), sb, X);
        O = mfma32(ld16(slot + C::OFF_R + s * 1024 + lane * 16), sb, O);
    }
    const bf16x4 vf = ld8(slot + C::OFF_V + wave * 512 + lane * 8);
    f32x4 U = mfma16(ld8(slot + C::OFF_NBKH + lane * 8), vf, zero4());
    U = mfma16(ld8(slot + C::OFF_NBKL + lane * 8), vf, U);
    U = mfma16(ld8(slot + C::OFF_TINV + lane * 8), cvt4(X), U);
    const bf16x4 ub = cvt4(U);
    O = mfma16(ld8(slot + C::OFF_MRKH + lane * 8), vf, O);
    O = mfma16(ld8(slot + C::OFF_MRKL + lane * 8), vf, O);
    O = mfma16(ld8(slot + C::OFF_MRA + lane * 8), ub, O);
#pragma unroll
    for (int q = 0; q < C::NRT; ++q) {
        const f32x4 eg = *(const f32x4 *)(slot + C::OFF_EGL + (16 * q + 4 * g) * 4);
        f32x4 acc = S[q] * eg;
        acc = mfma16(ld8(slot + C::OFF_KTH + q * 512 + lane * 8), vf, acc);
        acc = mfma16(ld8(slot + C::OFF_KTL + q * 512 + lane * 8), vf, acc);
        acc = mfma16(ld8(slot + C::OFF_AT + q * 512 + lane * 8), ub, acc);
        S[q] = acc;
    }
    const int col = wave * 16 + j;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = chunk * 16 + 4 * g + i;
        if (tok < T) o[(((size_t)bb * T + tok) * H + h) * D + col] = f32_to_bf16_bits(O[i]);
    }
}

template <int D>
__global__ __launch_bounds__(CK<D>::NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunked_kernel(
    int T, int H, const uint16_t *__restrict__ r, const uint16_t *__restrict__ w,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const uint16_t *__restrict__ a,
    const uint16_t *__restrict__ b, const float *__restrict__ s0, const uint8_t *__restrict__ mask,
    uint16_t *__restrict__ o, float *__restrict__ sf)
{
    using C = CK<D>;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int bh = blockIdx.x;
    const int bb = bh / H, h = bh % H;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int g = lane >> 4, j = lane & 15;
    const uint16_t *src[6] = {r, w, k, a, b, v};

    // Selection fragments: element e of lane (g, n) is 1 where channel
    // 4g + (e & 3) + 16 (e >> 2) of a block equals 16 hh + n.
    bf16x8 psel[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            psel[hh][e] = (__bf16)(((e >> 2) == hh && 4 * g + (e & 3) == j) ? 1.0f : 0.0f);

    // State tile: rows 16q + 4g + i, column 16 * wave + j.
    f32x4 S[C::NRT];
    const size_t st_base = (size_t)bh * D * D;
#pragma unroll
    for (int q = 0; q < C::NRT; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[q][i] = s0 ? s0[st_base + (size_t)(16 * q + 4 * g + i) * D + 16 * wave + j] : 0.0f;

    const int nchunks = (T + 15) / 16;
    RawTile<D> cur;
    if (wave < C::NP) load_raw<D>(cur, src, mask, T, H, bb, h, wave, lane);
    for (int c0 = 0; c0 < nchunks; c0 += C::NP) {
        if (wave < C::NP && c0 + wave < nchunks) precompute<D>(cur, lds + wave * C::SLOT, lane, psel);
        __syncthreads();
        if (wave < C::NP && c0 + C::NP + wave < nchunks)
            load_raw<D>(cur, src, mask, T, H, bb, h, c0 + C::NP + wave, lane);
#pragma unroll 1
        for (int p = 0; p < C::NP; ++p) {
            const int c = c0 + p;
            if (c >= nchunks) break;
            const char *slot = lds + p * C::SLOT;
            if (*(const int *)(slot + C::OFF_FLAG))
                chunk_exact<D>(S, r, w, k, v, a, b, mask, o, T, H, bb, h, c, wave, lane);
            else
                chunk_serial<D>(S, slot, o, T, H, bb, h, c, wave, lane);
        }
        __syncthreads();
    }

    if (sf) {
#pragma unroll
        for (int q = 0; q < C::NRT; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sf[st_base + (size_t)(16 * q + 4 * g + i) * D + 16 * wave + j] = S[q][i];
    }
}

// ===========================================================================
// Warp-specialised variant (K = V = 64).
//
// One workgroup of eight waves runs two (b, h) sequences.  Per sequence one
// wave is the consumer: it keeps the whole 64 x 64 fp32 state in MFMA
// accumulator registers and runs only the S-dependent chain.  Three waves
// are producers: producer p prepares chunks c = p, p + 3, ... from raw tiles
// that are streamed into a private LDS buffer with asynchronous global->LDS
// loads one chunk ahead, and hands the chunk's operands to the consumer
// through a three-slot LDS ring.  Hand-off uses LDS counters (ready[slot] =
// 2 (chunk + 1) + extreme-decay flag once a slot is filled; done = number of
// chunks whose operands the consumer has read), so producers and the
// consumer never meet at a workgroup barrier.  Every wait is bounded.
//
// Products on the consumer side pair operands along k so that each
// 16x16x32 MFMA carries two 16-token contractions, and the output is formed
// transposed (O^T = S^T R~^T + [U;V]^T [M_ra | M_rk]^T) so that each lane
// stores four adjacent bf16 outputs of one token.  The chunk-end decay is
// applied by the consumer after the rank-16 updates,
// S' = diag(e^{G_L}) (S + A^^T U + K^^T V), so that the producer hands over
// A^ and K^ (row-major token x channel tiles, read back as MFMA fragments
// with transposing LDS reads) instead of scaled, transposed copies.
// ===========================================================================

struct WS64 {
    static constexpr int D = 64;
    static constexpr int NCB = 2, NRT = 4, NCT = 4;   // channel blocks, row / column tiles
    static constexpr int NPROD = 3;                   // producers per sequence
    static constexpr int NSLOT = 3;
    static constexpr int NSEQ = 2;                    // sequences per workgroup
    static constexpr int NWAVE = NSEQ * (1 + NPROD);
    // slot layout (bytes); tiles are 16 tokens x 64 channels bf16, swizzled
    static constexpr int OFF_B = 0;                   // B~ frags, NCB x 1024
    static constexpr int OFF_R = 2048;                // R~ frags, NCB x 1024
    static constexpr int OFF_TN = 4096;               // [T | N_bk] A-frags, 1024
    static constexpr int OFF_MM = 5120;               // [M_ra^T | M_rk^T hi] B-frags, 1024
    static constexpr int OFF_MRKL = 6144;             // M_rk^T lo B-frag, 512
    static constexpr int OFF_EGL = 6656;              // e^{G_L}, 64 floats
    static constexpr int OFF_AH = 6912;               // A^ tile, 2048
    static constexpr int OFF_KH = 8960;               // K^ hi tile, 2048
    static constexpr int OFF_KL = 11008;              // K^ lo tile, 2048
    static constexpr int OFF_V = 13056;               // V tile, 2048 (global->LDS copy)
    static constexpr int SLOT = 15104;
    static constexpr int RAW = 5 * NCB * 1024;        // raw r, w, k, a, b tiles of one chunk
    static constexpr int OFF_SLOTS = 0;
};

constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ int lds_load_relaxed(int *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store_relaxed(int *p, int v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait until *p >= target; gives up after kSpinLimit polls so that a broken
// hand-off ends the kernel (with wrong results) instead of hanging it.
__device__ __forceinline__ int spin_ge(int *p, int target)
{
    int v = 0;
    for (int it = 0; it < kSpinLimit; ++it) {
        v = lds_load_relaxed(p);
        if (v >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    return v;
}

typedef __attribute__((address_space(3))) char *lds_ptr_t;

// Asynchronous 16-byte-per-lane global -> LDS copy: lane l's 16 bytes land at
// LDS byte address lds_base + 16 l.  Written out so that the compiler does not
// treat every later LDS access as dependent on it (it would insert a wait for
// all outstanding loads before each one); the copy has no register result, and
// every reader of the destination waits with an explicit s_waitcnt vmcnt(0).
__device__ __forceinline__ void copy16_to_lds(const void *gptr, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gptr), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const char *p)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_ptr_t)p);
}

// Producer: stream the raw r, w, k, a, b tiles of `chunk` into `raw`
// (5 arrays x NCB blocks, 1 KB each).  Lane l of each load fetches the 16 bytes of token l%16,
// channels 32s + 8(l/16) .. +7; tokens past T read token T-1 (discarded).
__device__ __forceinline__ void ws_issue_raw(uint32_t raw_lds, const uint16_t *const *src,
                                             size_t seq_base, uint32_t tok_stride, int T, int chunk,
                                             int lane)
{
    const int t = lane & 15, v = lane >> 4;
    const uint32_t tok = (uint32_t)min(chunk * 16 + t, T - 1);
    const size_t base = seq_base + (size_t)tok * tok_stride + 8 * v;
#pragma unroll
    for (int arr = 0; arr < 5; ++arr)
#pragma unroll
        for (int s = 0; s < WS64::NCB; ++s)
            copy16_to_lds(src[arr] + base + 32 * s, raw_lds + (arr * WS64::NCB + s) * 1024);
}

// Producer: read the staged raw tile into the register layout used by the
// precompute (lane (t, g): channels 32s + 16hh + 4g .. +3 of token t).
__device__ __forceinline__ void ws_read_raw(RawTile<64> &rt, const char *raw, int lane)
{
    const int t = lane & 15, g = lane >> 4;
#pragma unroll
    for (int arr = 0; arr < 5; ++arr)
#pragma unroll
        for (int s = 0; s < WS64::NCB; ++s)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                rt.x[s][arr][hh] = *(const u32x2 *)(raw + (arr * WS64::NCB + s) * 1024 +
                                                    16 * (t + 16 * (2 * hh + (g >> 1))) + 8 * (g & 1));
}

// Swizzled 16 x 64 bf16 tile: the 16-byte chunk c (channels 8c .. 8c + 7) of
// row r is stored at chunk position 8 r + (c ^ (r & 7)).  Row writes (one
// row per lane group) and transposing column reads (four rows per 16-lane
// group) then spread over all LDS banks.  Byte offset of the four channels
// col .. col + 3 (col a multiple of 4) of row r:
__device__ __forceinline__ int tile_off(int r, int col)
{
    return (r * 8 + ((col >> 3) ^ (r & 7))) * 16 + (col & 4) * 2;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// l supplies the address of four consecutive elements; lanes 4k .. 4k + 3
// together describe row k of a 4 x 16 block, and lane l receives column l.
// Here the group reads rows row0 .. row0 + 3, columns col0 .. col0 + 15 of
// a swizzled tile, so lane l gets X[row0 + k][col0 + l], k = 0..3: an MFMA
// B-fragment of X (k = token) or A-fragment of X^T.
__device__ __forceinline__ bf16x4 tile_tr(const char *tile, int row0, int col0, int lane)
{
    typedef __attribute__((address_space(3))) bf16x4 *lds_bf16x4_ptr;
    const int l = lane & 15;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_ptr)(tile + tile_off(row0 + (l >> 2), col0 + 4 * (l & 3))));
}

// Producer: copy the chunk's value tile (16 tokens x 64 channels) into the
// swizzled tile at LDS byte address `tile_lds` with two asynchronous
// global->LDS loads; lane l of load j fills chunk position 64 j + l.  Tokens
// past T read token T-1: a token that does not update has k = 0, so its
// value row is multiplied by zero everywhere.
__device__ __forceinline__ void ws_issue_v(uint32_t tile_lds, const uint16_t *v, size_t seq_base,
                                           uint32_t tok_stride, int T, int chunk, int lane)
{
#pragma unroll
    for (int jl = 0; jl < 2; ++jl) {
        const int row = 8 * jl + (lane >> 3);
        const int c = (lane & 7) ^ (row & 7);
        const uint32_t tok = (uint32_t)min(chunk * 16 + row, T - 1);
        copy16_to_lds(v + seq_base + (size_t)tok * tok_stride + 8 * c, tile_lds + 1024 * jl);
    }
}

// Producer: prepare one chunk's operands into `slot` (layout WS64).
//
// The per-channel decay prefix G_t = sum_{m<=t} w_m is formed on the matrix
// cores: w is first transposed to a token-contiguous fragment (selection
// MFMA, exact), then multiplied by the 16x16 upper-triangular ones matrix
// (`ltri`), which yields G in the same register layout as r, k, a, b.
// Precision: the r.k matrix M_rk (whose entries multiply the value tile
// directly in the output) is formed from hi/lo bf16 splits of both operands
// (three products, relative error about 2^-16); the other chunk matrices are
// single bf16 products with fp32 accumulation.  K^ is handed over as a hi/lo
// pair, as is M_rk, since both multiply the value tile.
// Returns the wave-uniform extreme-decay flag of the chunk.
__device__ int ws_precompute(const RawTile<64> &rt, char *slot, int lane, const bf16x8 *psel,
                             bf16x4 ltri)
{
    using C = WS64;
    const int t = lane & 15, g = lane >> 4;
    f32x4 mraT = zero4(), mrkT0 = zero4(), mrkT1 = zero4(), mba = zero4(), mbaT = zero4(), mbk = zero4();
    float emin = 1.0f;
    // Positive w (signed 16-bit view of the bf16 bits > 0) leaves the fast path.
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    s16x2 wmax = {(short)0x8000, (short)0x8000};
#pragma unroll
    for (int s = 0; s < C::NCB; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            wmax = __builtin_elementwise_max(wmax, __builtin_bit_cast(s16x2, rt.x[s][1][hh][0]));
            wmax = __builtin_elementwise_max(wmax, __builtin_bit_cast(s16x2, rt.x[s][1][hh][1]));
        }

    // Decay prefixes for all four 16-channel tiles (element e = 4hh + i of
    // block s holds channel 32s + 16hh + 4g + i of token t).
    f32x4 Gq[C::NCB][2];
#pragma unroll
    for (int s = 0; s < C::NCB; ++s) {
        const u32x4 wbits = {rt.x[s][1][0][0], rt.x[s][1][0][1], rt.x[s][1][1][0], rt.x[s][1][1][1]};
        const bf16x8 wb = __builtin_bit_cast(bf16x8, wbits);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            Gq[s][hh] = mfma16(cvt4(mfma32(wb, psel[hh], zero4())), ltri, zero4());
    }

#pragma unroll
    for (int s = 0; s < C::NCB; ++s) {
        float rv[8], kv[8], av[8], bv[8];
        unpack8(rt.x[s][0], rv);
        unpack8(rt.x[s][2], kv);
        unpack8(rt.x[s][3], av);
        unpack8(rt.x[s][4], bv);
        float Rt[8], Bt[8], Ah[8], Kh[8];
        f32x4 eGL4[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float G2 = Gq[s][e >> 2][e & 3] * 1.4426950408889634f;
            const float eG = __builtin_amdgcn_exp2f(G2);
            const float enG = __builtin_amdgcn_exp2f(-G2);
            const float eGp = row_shr<1>(eG, 1.0f);
            const float eGL = row_bcast15(eG);
            eGL4[e >> 2][e & 3] = eGL;
            emin = fminf(emin, eGL);
            Rt[e] = rv[e] * eG;
            Bt[e] = bv[e] * eGp;
            Ah[e] = av[e] * enG;
            Kh[e] = kv[e] * enG;
        }
        // e^{G_L} of channels 32s + 16hh + 4g .. +3 (one writer per row).
        if (t == 0) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                *(f32x4 *)(slot + C::OFF_EGL + (32 * s + 16 * hh + 4 * g) * 4) = eGL4[hh];
        }
        const bf16x8 Rh = pack8(Rt), Bh = pack8(Bt), Khh = pack8(Kh), Ahh = pack8(Ah);
        // (R~ K^^T)^T to about 16 bits: hi.hi + hi.lo + lo.hi.
        bf16x8 Rl, Khl;
        {
            float rem[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) rem[e] = Rt[e] - (float)Rh[e];
            Rl = pack8(rem);
#pragma unroll
            for (int e = 0; e < 8; ++e) rem[e] = Kh[e] - (float)Khh[e];
            Khl = pack8(rem);
        }
        mrkT0 = mfma32(Khh, Rh, mrkT0);
        mrkT1 = mfma32(Khh, Rl, mrkT1);
        mrkT1 = mfma32(Khl, Rh, mrkT1);

        mraT = mfma32(Ahh, Rh, mraT);   // (R~ A^^T)^T
        mba = mfma32(Bh, Ahh, mba);     // B~ A^^T
        mbaT = mfma32(Ahh, Bh, mbaT);   // (B~ A^^T)^T
        mbk = mfma32(Bh, Khh, mbk);     // B~ K^^T

        st16(slot + C::OFF_B + s * 1024 + lane * 16, Bh);
        st16(slot + C::OFF_R + s * 1024 + lane * 16, Rh);
        // Row t of the A^, K^ hi and K^ lo tiles, channels 32s + 16hh + 4g .. +3.
        const u32x4 ab = __builtin_bit_cast(u32x4, Ahh), kb = __builtin_bit_cast(u32x4, Khh),
                    lb = __builtin_bit_cast(u32x4, Khl);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int off = tile_off(t, 32 * s + 16 * hh + 4 * g);
            *(u32x2 *)(slot + C::OFF_AH + off) = u32x2{ab[2 * hh], ab[2 * hh + 1]};
            *(u32x2 *)(slot + C::OFF_KH + off) = u32x2{kb[2 * hh], kb[2 * hh + 1]};
            *(u32x2 *)(slot + C::OFF_KL + off) = u32x2{lb[2 * hh], lb[2 * hh + 1]};
        }
    }
    f32x4 mrkT = mrkT0 + mrkT1;

    const int j = lane & 15;
    f32x4 eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        mba[i] = row > j ? mba[i] : 0.0f;
        mbk[i] = row > j ? mbk[i] : 0.0f;
        mbaT[i] = j > row ? mbaT[i] : 0.0f;
        mraT[i] = j >= row ? mraT[i] : 0.0f;
        mrkT[i] = j >= row ? mrkT[i] : 0.0f;
        eye[i] = row == j ? 1.0f : 0.0f;
    }
    const bf16x4 n1 = cvt4(mba), n1t = cvt4(mbaT);
    const f32x4 p2 = mfma16(n1t, n1, zero4()), p2t = mfma16(n1, n1t, zero4());
    const bf16x4 n2 = cvt4(p2), n2t = cvt4(p2t);
    const f32x4 p4 = mfma16(n2t, n2, zero4()), p4t = mfma16(n2, n2t, zero4());
    const bf16x4 n4 = cvt4(p4), n4t = cvt4(p4t);
    const bf16x4 n8t = cvt4(mfma16(n4, n4t, zero4()));
    const f32x4 t1 = eye + mba, t1t = eye + mbaT;
    const bf16x4 t1b = cvt4(t1);
    const f32x4 t2 = mfma16(n2t, t1b, t1), t2t = mfma16(t1b, n2t, t1t);
    const bf16x4 t2b = cvt4(t2);
    const f32x4 t4 = mfma16(n4t, t2b, t2), t4t = mfma16(t2b, n4t, t2t);
    const bf16x4 tinv = cvt4(mfma16(cvt4(t4), n8t, t4t));
    st8(slot + C::OFF_TN + lane * 16, tinv);
    st8(slot + C::OFF_TN + lane * 16 + 8, cvt4(mfma16(cvt4(mbk), tinv, zero4())));
    st8(slot + C::OFF_MM + lane * 16, cvt4(mraT));
    bf16x4 hi, lo;
    split4(mrkT, hi, lo);
    st8(slot + C::OFF_MM + lane * 16 + 8, hi);
    st8(slot + C::OFF_MRKL + lane * 8, lo);
    return __any((int)(emin < kMinChunkFactor || wmax[0] > 0 || wmax[1] > 0)) ? 1 : 0;
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b)
{
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Consumer, exact path: token-by-token fp32 update of the whole state.
__device__ void ws_chunk_exact(f32x4 (*S)[4], const uint16_t *r, const uint16_t *w,
                               const uint16_t *k, const uint16_t *v, const uint16_t *a,
                               const uint16_t *b, const uint8_t *mask, uint16_t *o, int T, int H,
                               int bb, int h, int chunk, int lane)
{
    constexpr int D = 64;
    const int g = lane >> 4, j = lane & 15;
    for (int tt = 0; tt < 16; ++tt) {
        const int tok = chunk * 16 + tt;
        if (tok >= T) break;
        const bool upd = mask == nullptr || mask[(size_t)bb * T + tok] != 0;
        const size_t base = (((size_t)bb * T + tok) * H + h) * D;
        if (upd) {
            float sb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 bq = *(const u32x2 *)(b + base + 16 * q + 4 * g);
                const float be[4] = {bf16_lo(bq[0]), bf16_hi(bq[0]), bf16_lo(bq[1]), bf16_hi(bq[1])};
#pragma unroll
                for (int n = 0; n < 4; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sb[n] = fmaf(be[i], S[q][n][i], sb[n]);
            }
#pragma unroll
            for (int n = 0; n < 4; ++n) sb[n] = xor_sum(xor_sum(sb[n], 16), 32);
            float vj[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) vj[n] = bf16_bits_to_f32(v[base + 16 * n + j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 wq = *(const u32x2 *)(w + base + 16 * q + 4 * g);
                const u32x2 aq = *(const u32x2 *)(a + base + 16 * q + 4 * g);
                const u32x2 kq = *(const u32x2 *)(k + base + 16 * q + 4 * g);
                const float we[4] = {bf16_lo(wq[0]), bf16_hi(wq[0]), bf16_lo(wq[1]), bf16_hi(wq[1])};
                const float ae[4] = {bf16_lo(aq[0]), bf16_hi(aq[0]), bf16_lo(aq[1]), bf16_hi(aq[1])};
                const float ke[4] = {bf16_lo(kq[0]), bf16_hi(kq[0]), bf16_lo(kq[1]), bf16_hi(kq[1])};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d = __expf(we[i]);
#pragma unroll
                    for (int n = 0; n < 4; ++n)
                        S[q][n][i] = fmaf(d, S[q][n][i], fmaf(ae[i], sb[n], ke[i] * vj[n]));
                }
            }
        }
        float ov[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x2 rq = *(const u32x2 *)(r + base + 16 * q + 4 * g);
            const float re[4] = {bf16_lo(rq[0]), bf16_hi(rq[0]), bf16_lo(rq[1]), bf16_hi(rq[1])};
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[n] = fmaf(re[i], S[q][n][i], ov[n]);
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) ov[n] = xor_sum(xor_sum(ov[n], 16), 32);
        if (g == 0) {
#pragma unroll
            for (int n = 0; n < 4; ++n) o[base + 16 * n + j] = f32_to_bf16_bits(ov[n]);
        }
    }
}

// Consumer: the S-dependent part of one chunk for all 64 columns.  Work is
// issued in dependency order across the four independent column tiles, and
// the S-independent products are placed where they fill the latency of the
// S -> X -> U -> S' chain.
// Store one chunk's output tile held as O^T fragments (lane (g, t): token t,
// columns 16n + 4g .. +3).
__device__ __forceinline__ void ws_store_out(const f32x4 *Ot, uint16_t *o, int T, int H, int bb, int h,
                                             int chunk, int lane)
{
    const int g = lane >> 4, t = lane & 15;
    const int tok = chunk * 16 + t;
    if (chunk >= 0 && tok < T) {
        uint16_t *op = o + (((size_t)bb * T + tok) * H + h) * 64 + 4 * g;
#pragma unroll
        for (int n = 0; n < 4; ++n)
            *(u32x2 *)(op + 16 * n) = u32x2{cvt2_bits(Ot[n][0], Ot[n][1]), cvt2_bits(Ot[n][2], Ot[n][3])};
    }
}

__device__ __forceinline__ void ws_chunk_serial(f32x4 (*S)[4], const char *slot, uint16_t *o, int T,
                                                int H, int bb, int h, int chunk, int lane)
{
    using C = WS64;
    const int g = lane >> 4;
    bf16x8 sb0[4], sb1[4];
    bf16x4 vf[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        sb0[n] = cat8(cvt4(S[0][n]), cvt4(S[1][n]));
        sb1[n] = cat8(cvt4(S[2][n]), cvt4(S[3][n]));
        vf[n] = tile_tr(slot + C::OFF_V, 4 * g, 16 * n, lane);   // V[4g + i][16n + j]
    }
    const bf16x8 bt0 = ld16(slot + C::OFF_B + lane * 16), bt1 = ld16(slot + C::OFF_B + 1024 + lane * 16);
    // X = B~ S
    f32x4 X[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) X[n] = mfma32(bt0, sb0[n], zero4());
    // S += K^lo^T V  (independent of X; the decay is applied at the end)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bf16x4 ktl = tile_tr(slot + C::OFF_KL, 4 * g, 16 * q, lane);
#pragma unroll
        for (int n = 0; n < 4; ++n) S[q][n] = mfma16(ktl, vf[n], S[q][n]);
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) X[n] = mfma32(bt1, sb1[n], X[n]);
    // O^T, S-part (old S)
    const bf16x8 rt0 = ld16(slot + C::OFF_R + lane * 16), rt1 = ld16(slot + C::OFF_R + 1024 + lane * 16);
    const bf16x4 mrkl = ld8(slot + C::OFF_MRKL + lane * 8);
    f32x4 Ot[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) Ot[n] = mfma32(sb0[n], rt0, zero4());
    // U = T X + N_bk V
    const bf16x8 tn = ld16(slot + C::OFF_TN + lane * 16);
    bf16x8 uv[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) uv[n] = cat8(cvt4(mfma32(tn, cat8(cvt4(X[n]), vf[n]), zero4())), vf[n]);
#pragma unroll
    for (int n = 0; n < 4; ++n) Ot[n] = mfma32(sb1[n], rt1, Ot[n]);
#pragma unroll
    for (int n = 0; n < 4; ++n) Ot[n] = mfma16(vf[n], mrkl, Ot[n]);
    // S <- diag(e^{G_L}) (S + [A^^T | K^hi^T] [U; V])
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bf16x8 atk = cat8(tile_tr(slot + C::OFF_AH, 4 * g, 16 * q, lane),
                                tile_tr(slot + C::OFF_KH, 4 * g, 16 * q, lane));
        const f32x4 eg = *(const f32x4 *)(slot + C::OFF_EGL + (16 * q + 4 * g) * 4);
#pragma unroll
        for (int n = 0; n < 4; ++n) S[q][n] = mfma32(atk, uv[n], S[q][n]) * eg;
    }
    // O^T += [U; V]^T [M_ra | M_rk]^T
    const bf16x8 mm = ld16(slot + C::OFF_MM + lane * 16);
#pragma unroll
    for (int n = 0; n < 4; ++n) Ot[n] = mfma32(uv[n], mm, Ot[n]);
    ws_store_out(Ot, o, T, H, bb, h, chunk, lane);
}

__global__ __launch_bounds__(64 * WS64::NWAVE) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunked64_ws_kernel(
    int T, int H, int nbh, const uint16_t *__restrict__ r, const uint16_t *__restrict__ w,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const uint16_t *__restrict__ a,
    const uint16_t *__restrict__ b, const float *__restrict__ s0, const uint8_t *__restrict__ mask,
    uint16_t *__restrict__ o, float *__restrict__ sf)
{
    using C = WS64;
    // Separate LDS objects: the compiler must wait for outstanding
    // global->LDS loads before touching the object they write (the raw
    // buffers), but not before the slot rings or the hand-off counters.
    __shared__ __attribute__((aligned(16))) char lds_slots[C::NSEQ * C::NSLOT * C::SLOT];
    __shared__ __attribute__((aligned(16))) char lds_raw[C::NSEQ * C::NPROD * C::RAW];
    __shared__ int lds_sync[32];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int g = lane >> 4, j = lane & 15;
    const int nchunks = (T + 15) / 16;

    // Role assignment by SIMD placement.  The consumers (mostly MFMA work,
    // slowed down by sharing a SIMD with VALU-heavy producers) are taken
    // from the SIMDs with the fewest workgroup waves, at most one per SIMD
    // while that is possible.  The other waves become producers, alternating
    // between the sequences in (SIMD, wave) order so that each sequence's
    // producers are spread over different SIMDs.  (Measured: eight waves
    // with three producers per sequence beat six waves with two, where the
    // consumers run alone on a SIMD but production falls behind.)
    // Correctness does not depend on the placement; it only picks which wave
    // does what.
    int *key_of = lds_sync + 16;   // NWAVE entries
    if (threadIdx.x < 16) lds_sync[threadIdx.x] = 0;
    if (lane == 0) {
        unsigned hw;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        key_of[wave] = (int)((hw >> 4) & 3) * 8 + wave;   // unique key: (simd, wave)
    }
    __syncthreads();
    int ckey[C::NWAVE];   // (rank on the SIMD, waves on the SIMD, SIMD, wave)
#pragma unroll
    for (int w1 = 0; w1 < C::NWAVE; ++w1) {
        int n = 0, before = 0;
#pragma unroll
        for (int w2 = 0; w2 < C::NWAVE; ++w2) {
            const bool same = (key_of[w2] >> 3) == (key_of[w1] >> 3);
            n += same ? 1 : 0;
            before += (same && key_of[w2] < key_of[w1]) ? 1 : 0;
        }
        ckey[w1] = (before * 16 + n) * 32 + key_of[w1];
    }
    int crank = 0, prank = 0;
#pragma unroll
    for (int w2 = 0; w2 < C::NWAVE; ++w2) crank += ckey[w2] < ckey[wave] ? 1 : 0;
    const bool is_cons = crank < C::NSEQ;
#pragma unroll
    for (int w2 = 0; w2 < C::NWAVE; ++w2) {
        int cr = 0;
#pragma unroll
        for (int w3 = 0; w3 < C::NWAVE; ++w3) cr += ckey[w3] < ckey[w2] ? 1 : 0;
        prank += (cr >= C::NSEQ && key_of[w2] < key_of[wave]) ? 1 : 0;
    }
    const int seq = is_cons ? crank : prank % C::NSEQ;
    const int role = is_cons ? 0 : 1 + prank / C::NSEQ;   // 0 = consumer, 1.. = producers
    const int bh = blockIdx.x * C::NSEQ + seq;
    if (bh >= nbh) return;
    const int bb = bh / H, h = bh % H;
    char *const lds = lds_slots + seq * C::NSLOT * C::SLOT;
    int *ready = lds_sync + 8 * seq;   // ready[NSLOT], then done
    int *done = ready + C::NSLOT;

    if (role == 0) {
        // ---------------- consumer ----------------
        f32x4 S[4][4];   // S[q][n]: rows 16q + 4g + i, column 16n + j
        const size_t st_base = (size_t)bh * 64 * 64;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[q][n][i] = s0 ? s0[st_base + (size_t)(16 * q + 4 * g + i) * 64 + 16 * n + j] : 0.0f;
        for (int c = 0; c < nchunks; ++c) {
            const char *slot = lds + C::OFF_SLOTS + (c % C::NSLOT) * C::SLOT;
            // ready[slot] = 2 (c + 1) + extreme-decay flag once chunk c is in the slot
            const int rv = spin_ge(&ready[c % C::NSLOT], 2 * (c + 1));
            if (rv & 1)
                ws_chunk_exact(S, r, w, k, v, a, b, mask, o, T, H, bb, h, c, lane);
            else
                ws_chunk_serial(S, slot, o, T, H, bb, h, c, lane);
            lds_wait();                          // all reads of the slot have returned
            lds_store_relaxed(done, c + 1);
        }
        if (sf) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int n = 0; n < 4; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sf[st_base + (size_t)(16 * q + 4 * g + i) * 64 + 16 * n + j] = S[q][n][i];
        }
    } else {
        // ---------------- producers ----------------
        const int p = role - 1;
        char *raw = lds_raw + (seq * C::NPROD + p) * C::RAW;
        const uint32_t raw_lds = lds_addr(raw);
        // Element offset of (bb, token 0, h, channel 0) and between tokens.
        const size_t seq_base = ((size_t)bb * T * H + h) * 64;
        const uint32_t tok_stride = (uint32_t)H * 64;
        const uint16_t *src[5] = {r, w, k, a, b};
        bf16x8 psel[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                psel[hh][e] = (__bf16)(((e >> 2) == hh && 4 * g + (e & 3) == j) ? 1.0f : 0.0f);
        // B-fragment of the inclusive prefix-sum matrix: [token' <= token].
        bf16x4 ltri;
#pragma unroll
        for (int i = 0; i < 4; ++i) ltri[i] = (__bf16)((4 * g + i <= j) ? 1.0f : 0.0f);
        // Loop-carried request for this producer's next chunk: the mask byte
        // of token (next chunk, lane & 15).
        uint32_t mnext = 1;
        const int t = lane & 15;
        if (p < nchunks) {
            ws_issue_raw(raw_lds, src, seq_base, tok_stride, T, p, lane);
            if (mask) mnext = mask[(size_t)bb * T + min(p * 16 + t, T - 1)];
        }
        for (int c = p; c < nchunks; c += C::NPROD) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            const uint32_t mcur = mnext;
            RawTile<64> rt;
            ws_read_raw(rt, raw, lane);
            lds_wait();
            if (c + C::NPROD < nchunks) {
                const int cn = c + C::NPROD;
                ws_issue_raw(raw_lds, src, seq_base, tok_stride, T, cn, lane);
                if (mask) mnext = mask[(size_t)bb * T + min(cn * 16 + t, T - 1)];
            }
            const int tok = c * 16 + t;
            rt.valid = tok < T;
            rt.upd = rt.valid && mcur != 0;
            zero_inactive<64>(rt, 5);
            char *slot = lds + C::OFF_SLOTS + (c % C::NSLOT) * C::SLOT;
            spin_ge(done, c - C::NSLOT + 1);   // the slot's previous chunk is consumed
            ws_issue_v(lds_addr(slot + C::OFF_V), v, seq_base, tok_stride, T, c, lane);
            if (!__all(rt.upd)) {
                // Value rows of tokens that do not update are cleared, so that
                // whatever they hold (even inf or nan) cannot reach the state.
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (!rt.upd) {
                    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        *(u32x4 *)(slot + C::OFF_V + tile_off(t, 16 * g + 8 * hh)) = zero;
                }
            }
            const int flag = ws_precompute(rt, slot, lane, psel, ltri);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the value tile has landed
            lds_wait();
            lds_store_relaxed(&ready[c % C::NSLOT], 2 * (c + 1) + flag);
        }
    }
}

template <int D>
static hipError_t launch_ck(const FwdArgs &p, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.B * p.H)), block(CK<D>::NT);
    hipLaunchKernelGGL((chunked_kernel<D>), grid, block, CK<D>::LDS, stream, p.T, p.H,
                       (const uint16_t *)p.r, (const uint16_t *)p.w, (const uint16_t *)p.k,
                       (const uint16_t *)p.v, (const uint16_t *)p.a, (const uint16_t *)p.b, p.s0,
                       p.mask, (uint16_t *)p.o, p.sf);
    return hipGetLastError();
}

static hipError_t launch_ws64(const FwdArgs &p, hipStream_t stream)
{
    const int nbh = p.B * p.H;
    const dim3 grid((unsigned)((nbh + WS64::NSEQ - 1) / WS64::NSEQ)), block(64 * WS64::NWAVE);
    hipLaunchKernelGGL(chunked64_ws_kernel, grid, block, 0, stream, p.T, p.H, nbh,
                       (const uint16_t *)p.r, (const uint16_t *)p.w, (const uint16_t *)p.k,
                       (const uint16_t *)p.v, (const uint16_t *)p.a, (const uint16_t *)p.b, p.s0,
                       p.mask, (uint16_t *)p.o, p.sf);
    return hipGetLastError();
}

hipError_t launch_chunked(const FwdArgs &p, hipStream_t stream)
{
    return p.D == 64 ? launch_ws64(p, stream) : launch_ck<128>(p, stream);
}

}  // namespace wkv7

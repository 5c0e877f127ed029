// Chunked WKV7 forward on bf16 MFMA (bf16 I/O, fp32 state), K = V = 64 or 128.
//
// The recurrence (rwkv-ops README, section "rwkv7op 使用方法", read as the
// generalized delta rule) is evaluated 16 tokens at a time.  Within a chunk
// with start state S (K x V, fp32), log-decay prefix G_i = sum_{m<=i} w_m and
// G_{-1} = 0 (per channel), u_i = b_i^T S_{i-1} unrolls to
//
//   U   = T (B~ S + M_bk V)                    T = (I - M_ba)^-1
//   O   = R~ S + M_ra U + M_rk V
//   S' = diag(e^{G_L}) (S + A^^T U + K^^T V)
//
// with  R~ = r e^{G},  B~ = b e^{G_{i-1}},  A^ = a e^{-G},  K^ = k e^{-G},
// M_ba = B~ A^^T and M_bk = B~ K^^T strictly lower, M_ra = R~ A^^T and
// M_rk = R~ K^^T lower with diagonal.  Every factor of the form e^{G_i - G_j}
// with j <= i is <= 1, and the split factors stay finite while the chunk's
// decay sum is above -60; chunks beyond that (or with w > 0) take an exact
// token-by-token path instead.  A token with mask 0 (or past T) gets
// w = a = k = b = 0, an exact identity step.
//
// Layout of the work (warp specialisation).  Per (b, h) sequence, consumer
// waves each keep a column slice of the fp32 state (64 columns at D = 64,
// 32 at D = 128) in MFMA accumulator registers and run only the
// S-dependent chain; the column split is exact (U, O and S' of a column
// slice depend only on that slice).
// Producer waves prepare chunks c = p, p + NPROD, ... from raw tiles streamed
// into a private LDS buffer with asynchronous global->LDS loads one chunk
// ahead, and hand each chunk's operands to the consumers through a ring of
// LDS slots.  Hand-off uses LDS counters (ready[slot] = 2 (chunk + 1) +
// extreme-decay flag once a slot is filled; done[i] = chunks consumer i has
// finished reading), so producers and consumers never meet at a workgroup
// barrier.  Every wait is bounded.  At D = 64 one workgroup runs two
// sequences of one consumer and three producers with three slots each (eight
// waves); at D = 128 one sequence of four consumers and four producers with
// two slots (eight waves).
//
// Products on the consumer side pair operands along k so that each
// 16x16x32 MFMA carries two 16-token contractions, and the output is formed
// transposed (O^T = S^T R~^T + [U;V]^T [M_ra | M_rk]^T) so that each lane
// stores four adjacent bf16 outputs of one token.  The producer hands over
// A^ and K^ as row-major token x channel tiles that the consumer reads back
// as MFMA fragments with transposing LDS reads; the chunk-end decay is
// applied by the consumer after the rank-16 updates.
//
// Precision.  MFMA operands are bf16 with fp32 accumulation.  The r.k matrix
// M_rk and K^, which multiply the exact-bf16 value tile, are carried as hi/lo
// bf16 pairs; the other chunk matrices are single bf16 products.
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace wkv7 {

// A chunk whose summed decay factor exp(G_L) falls below e^-60 in any channel
// would need factors up to e^60 in the split form; it takes the exact path.
constexpr float kMinChunkFactor = 8.75651076e-27f;   // e^-60

template <int D> struct WS {
    static_assert(D == 64 || D == 128, "head size");
    static constexpr int NCB = D / 32;                 // 32-channel blocks
    static constexpr int NQ = D / 16;                  // 16-row tiles of the state
    // D = 64: two sequences of one consumer (64 state columns) and three
    // producers, three slots each.  D = 128: one sequence of four consumers
    // (32 columns each, so that a 128 x 32 state slice and its working set
    // stay in ordinary VGPRs) and four producers, which leaves LDS for two
    // slots only: a chunk costs a producer about four times what it costs a
    // consumer, and a fourth producer (0.98 -> 0.875 ms on B16 T4096 H32)
    // is worth more than a third slot.  Two waves per SIMD in both cases.
    static constexpr int NCONS = D == 64 ? 1 : 4;      // consumers per sequence
    static constexpr int CW = D / NCONS;               // state columns per consumer
    static constexpr int NT = CW / 16;                 // 16-column tiles per consumer
    static constexpr int NPROD = D == 64 ? 3 : 4;      // producers per sequence
    static constexpr int NSLOT = D == 64 ? 3 : 2;      // slot ring depth per sequence
    static constexpr int NSEQ = D == 64 ? 2 : 1;       // sequences per workgroup
    static constexpr int NWAVE = NSEQ * (NCONS + NPROD);
    static constexpr int WAVES_PER_SIMD = (NWAVE + 3) / 4;
    static constexpr int TILE = 16 * D * 2;            // 16 tokens x D channels, bf16
    // slot layout (bytes); fragments are 64 lanes x 16 (or 8) bytes
    static constexpr int OFF_B = 0;                    // B~ A-frags, NCB x 1024
    static constexpr int OFF_R = OFF_B + NCB * 1024;   // R~ A-frags, NCB x 1024
    static constexpr int OFF_TN = OFF_R + NCB * 1024;  // [T | N_bk] A-frags, 1024
    static constexpr int OFF_MM = OFF_TN + 1024;       // [M_ra^T | M_rk^T hi] B-frags, 1024
    static constexpr int OFF_MRKL = OFF_MM + 1024;     // M_rk^T lo B-frag, 512
    static constexpr int OFF_EGL = OFF_MRKL + 512;     // e^{G_L}, D floats
    static constexpr int OFF_SIG = OFF_EGL + 4 * D;    // Gated DeltaNet output scale, 16 floats
    static constexpr int OFF_AH = (OFF_SIG + 64 + 255) / 256 * 256;   // A^ tile
    static constexpr int OFF_KH = OFF_AH + TILE;       // K^ hi tile
    static constexpr int OFF_KL = OFF_KH + TILE;       // K^ lo tile
    static constexpr int OFF_V = OFF_KL + TILE;        // V tile (global->LDS copy)
    static constexpr int SLOT = OFF_V + TILE;
    static constexpr int RAW = 5 * NCB * 1024;         // raw r, w, k, a, b tiles of one chunk
    static constexpr int LDS_SLOTS = NSEQ * NSLOT * SLOT;
    static constexpr int LDS_RAW = NSEQ * NPROD * RAW;
    static_assert(LDS_SLOTS + LDS_RAW + 128 <= 160 * 1024, "LDS budget");
};

// Raw bf16 tiles of one chunk in the precompute lane layout: lane (t = l%16,
// g = l/16) holds token t, channels 32s + 16hh + 4g .. +3 in x[s][arr][hh].
// Array order: r, w, k, a, b.
template <int D> struct RawTile {
    u32x2 x[D / 32][5][2];
    int upd;     // token updates the state
    int valid;   // token exists (t0 + t < T)
};

// Make a token that does not update an exact identity step: w, k, a and b
// are cleared, so that whatever they hold (even inf or nan) cannot reach the
// state; r stays, since such a token still emits an output.  A token past T
// is inert (r = 0 as well).
template <int D>
__device__ __forceinline__ void zero_inactive(RawTile<D> &rt)
{
    if (__all(rt.upd)) return;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int arr = 1; arr <= 4; ++arr)
                rt.x[s][arr][hh] = rt.upd ? rt.x[s][arr][hh] : u32x2{0u, 0u};
            rt.x[s][0][hh] = rt.valid ? rt.x[s][0][hh] : u32x2{0u, 0u};
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

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b)
{
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---- hand-off counters ------------------------------------------------------

__device__ __forceinline__ int lds_load_relaxed(int *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store_relaxed(int *p, int v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait until *p >= target, polling at most `limit` times.  Returns the last
// value read: a value below target means the wait gave up (a broken hand-off
// then ends the kernel instead of hanging it, and the caller poisons its
// results so that the failure is visible).  *flag is read with every poll
// (the sequence's failure flag, at no extra round trip).
__device__ __forceinline__ int spin_ge(int *p, int target, int limit, int *flag, int &flag_value)
{
    int v = 0, f = 0;
    for (int it = 0; it < limit; ++it) {
        v = lds_load_relaxed(p);
        f = lds_load_relaxed(flag);
        if (v >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    flag_value = f;
    return v;
}
// Wait until p[0..n) are all >= target (bounded like spin_ge); false if the
// wait gave up.
template <int N>
__device__ __forceinline__ bool spin_all_ge(int *p, int target, int limit)
{
    bool ok = false;
    for (int it = 0; it < limit; ++it) {
        int v = lds_load_relaxed(p);
#pragma unroll
        for (int i = 1; i < N; ++i) v = min(v, lds_load_relaxed(p + i));
        if (v >= target) {
            ok = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    return ok;
}

// ---- global -> LDS staging ----------------------------------------------------

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

// Producer: stream the raw r, w, k, a, b tiles of `chunk` into the LDS buffer
// at `raw_lds` (5 arrays x NCB blocks, 1 KB each).  Lane l of each load
// fetches the 16 bytes of token l%16, channels 32s + 8(l/16) .. +7; tokens
// past T read token T-1 (discarded).
template <int D, bool GDN>
__device__ __forceinline__ void ws_issue_raw(uint32_t raw_lds, const uint16_t *const *src,
                                             size_t seq_base, uint32_t tok_stride, int T, int chunk,
                                             int lane)
{
    const int t = lane & 15, v = lane >> 4;
    const uint32_t tok = (uint32_t)min(chunk * 16 + t, T - 1);
    const size_t base = seq_base + (size_t)tok * tok_stride + 8 * v;
#pragma unroll
    for (int arr = 0; arr < 5; ++arr) {
        if (GDN && arr != 0 && arr != 2) continue;   // Gated DeltaNet: q and k only
#pragma unroll
        for (int s = 0; s < WS<D>::NCB; ++s)
            copy16_to_lds(src[arr] + base + 32 * s, raw_lds + (arr * WS<D>::NCB + s) * 1024);
    }
}

// Producer: read the staged raw tile into the register layout used by the
// precompute (lane (t, g): channels 32s + 16hh + 4g .. +3 of token t).
template <int D, bool GDN>
__device__ __forceinline__ void ws_read_raw(RawTile<D> &rt, const char *raw, int lane)
{
    const int t = lane & 15, g = lane >> 4;
#pragma unroll
    for (int arr = 0; arr < 5; ++arr)
#pragma unroll
        for (int s = 0; s < WS<D>::NCB; ++s)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                rt.x[s][arr][hh] = (!GDN || arr == 0 || arr == 2)
                                       ? *(const u32x2 *)(raw + (arr * WS<D>::NCB + s) * 1024 +
                                                          16 * (t + 16 * (2 * hh + (g >> 1))) + 8 * (g & 1))
                                       : u32x2{0u, 0u};   // Gated DeltaNet: unused
}

// Gated DeltaNet (rwkv-ops README, section "gdn_recurrent 使用方法": q, k
// L2-normalised inside, g a log-space gate, beta a write strength), read as
// the gated delta rule S = e^g (I - beta kn kn^T) S + beta kn v^T, o = S^T qn,
// is the generalized delta rule with
//   r = qn,  w = g (every channel),  k = beta kn,  a = -e^g beta kn,  b = kn.
// Each of r, k, a, b is a raw bf16 input (q or k) times a per-token scalar,
// so the producer keeps q and k as loaded and hands the precompute the four
// scalars: they are applied in fp32 together with the decay factors, before
// the one rounding to bf16 that the MFMA operands take anyway (rounding
// qn, beta kn, ... to bf16 first would add a second rounding, which costs
// about half of the bf16 error budget on random q and k).
// Producer: gate into the w slot (every channel) and the token's scalars
// sc = {1/|q|, beta/|k|, -e^g beta/|k|, 1/|k|} (norms with 1e-6 added to the
// squared length).  The four lanes of a token (t, t + 16, t + 32, t + 48)
// together hold its D channels.
template <int D>
__device__ __forceinline__ void gdn_scalars(RawTile<D> &rt, uint32_t gbits, float beta, float *sc)
{
    constexpr int NCB = D / 32;
    float nq = 0.0f, nk = 0.0f;
#pragma unroll
    for (int s = 0; s < NCB; ++s) {
        float qv[8], kv[8];
        unpack8(rt.x[s][0], qv);
        unpack8(rt.x[s][2], kv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            nq = fmaf(qv[e], qv[e], nq);
            nk = fmaf(kv[e], kv[e], nk);
        }
    }
    nq = xsum32(xsum16(nq));
    nk = xsum32(xsum16(nk));
    const float iq = 1.0f / sqrtf(nq + 1e-6f), ik = 1.0f / sqrtf(nk + 1e-6f);
    const float gate = bf16_bits_to_f32((uint16_t)gbits);
    sc[0] = iq;
    sc[1] = beta * ik;
    sc[2] = -__expf(gate) * beta * ik;
    sc[3] = ik;
    const uint32_t w2 = (gbits & 0xffffu) | (gbits << 16);
#pragma unroll
    for (int s = 0; s < NCB; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) rt.x[s][1][hh] = u32x2{w2, w2};
}

// Swizzled 16 x D bf16 tile: the 16-byte chunk c (channels 8c .. 8c + 7) of
// row r is stored at chunk position (D/8) r + (c ^ (r & 7)).  Row writes (one
// row per lane group) and transposing column reads (four rows per 16-lane
// group) then spread over all LDS banks.  Byte offset of the four channels
// col .. col + 3 (col a multiple of 4) of row r:
template <int D>
__device__ __forceinline__ int tile_off(int r, int col)
{
    return (r * (D / 8) + ((col >> 3) ^ (r & 7))) * 16 + (col & 4) * 2;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// l supplies the address of four consecutive elements; lanes 4k .. 4k + 3
// together describe row k of a 4 x 16 block, and lane l receives column l.
// Here the group reads rows row0 .. row0 + 3, columns col0 .. col0 + 15 of
// a swizzled tile, so lane l gets X[row0 + k][col0 + l], k = 0..3: an MFMA
// B-fragment of X (k = token) or A-fragment of X^T.
template <int D>
__device__ __forceinline__ bf16x4 tile_tr(const char *tile, int row0, int col0, int lane)
{
    typedef __attribute__((address_space(3))) bf16x4 *lds_bf16x4_ptr;
    const int l = lane & 15;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_ptr)(tile + tile_off<D>(row0 + (l >> 2), col0 + 4 * (l & 3))));
}

// Producer: copy the chunk's value tile (16 tokens x D channels) into the
// swizzled tile at LDS byte address `tile_lds` with D/32 asynchronous
// global->LDS loads; lane l of load j fills chunk position 64 j + l.  Tokens
// past T read token T-1: a token that does not update has k = 0 and b = 0,
// so its value row is multiplied by zero everywhere (and rows of masked
// tokens are cleared outright before the slot is handed over).
template <int D>
__device__ __forceinline__ void ws_issue_v(uint32_t tile_lds, const uint16_t *v, size_t seq_base,
                                           uint32_t tok_stride, int T, int chunk, int lane)
{
#pragma unroll
    for (int jl = 0; jl < D / 32; ++jl) {
        const int pos = 64 * jl + lane;
        const int row = pos / (D / 8);
        const int c = (pos % (D / 8)) ^ (row & 7);
        const uint32_t tok = (uint32_t)min(chunk * 16 + row, T - 1);
        copy16_to_lds(v + seq_base + (size_t)tok * tok_stride + 8 * c, tile_lds + 1024 * jl);
    }
}

// ---- producer: one chunk's operands -----------------------------------------
//
// The per-channel decay prefix G_t = sum_{m<=t} w_m is formed on the matrix
// cores: w is first transposed to a token-contiguous fragment (selection
// MFMA, exact), then multiplied by the 16x16 upper-triangular ones matrix
// (`ltri`), which yields G in the same register layout as r, k, a, b.
// Precision: M_rk is formed from hi/lo bf16 splits of both operands (three
// products, relative error about 2^-16) and handed over as a hi/lo pair, as
// is K^; the other chunk matrices are single bf16 products with fp32
// accumulation.  T = (I - M_ba)^-1 uses the nilpotent doubling product
// (I + N^8)(I + N^4)(I + N^2)(I + N), every factor kept both as X and X^T
// (MFMA accumulators of X^T are the A-fragments of X).
// Everything is formed in registers first (ChunkOps) and written to the slot
// afterwards, so that a producer only needs its slot back for the short write.
template <int D> struct ChunkOps {
    bf16x8 B[D / 32], R[D / 32];        // B~, R~ A-fragments per 32-channel block
    u32x4 ah[D / 32], kh[D / 32], kl[D / 32];   // row t of the A^, K^ hi, K^ lo tiles
    f32x4 egl[D / 32][2];               // e^{G_L} of channels 32s + 16hh + 4g .. +3
    bf16x4 tinv, tnbk, mra, mrkh, mrkl;
    float sig;                          // Gated DeltaNet: e^{G_t} / |q_t| of token t
    int flag;                           // wave-uniform extreme-decay flag
};

// sc: per-token scalars of r, k, a, b (Gated DeltaNet only; see gdn_scalars).
template <int D, bool GDN>
__device__ void ws_precompute(const RawTile<D> &rt, ChunkOps<D> &op, int lane, const bf16x8 *psel,
                              bf16x4 ltri, const float *sc)
{
    using C = WS<D>;
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

#pragma unroll
    for (int s = 0; s < C::NCB; ++s) {
        // Decay prefix of block s (element e = 4hh + i holds channel
        // 32s + 16hh + 4g + i of token t).
        f32x4 Gq[2];
        {
            const u32x4 wbits = {rt.x[s][1][0][0], rt.x[s][1][0][1], rt.x[s][1][1][0], rt.x[s][1][1][1]};
            const bf16x8 wb = __builtin_bit_cast(bf16x8, wbits);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                Gq[hh] = mfma16(cvt4(mfma32(wb, psel[hh], zero4())), ltri, zero4());
        }
        float rv[8], kv[8], av[8], bv[8];
        unpack8(rt.x[s][0], rv);
        unpack8(rt.x[s][2], kv);
        if constexpr (!GDN) {
            unpack8(rt.x[s][3], av);
            unpack8(rt.x[s][4], bv);
        }
        float Rt[8], Bt[8], Ah[8], Kh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float G2 = Gq[e >> 2][e & 3] * 1.4426950408889634f;
            const float eG = __builtin_amdgcn_exp2f(G2);
            const float enG = __builtin_amdgcn_exp2f(-G2);
            const float eGp = row_shr<1>(eG, 1.0f);
            const float eGL = row_bcast15(eG);
            op.egl[s][e >> 2][e & 3] = eGL;
            emin = fminf(emin, eGL);
            if constexpr (GDN) {
                if (s == 0 && e == 0) op.sig = eG * sc[0];   // the gate is the same on every channel
                Rt[e] = rv[e] * (eG * sc[0]);
                Kh[e] = kv[e] * (enG * sc[1]);
                Ah[e] = kv[e] * (enG * sc[2]);
                Bt[e] = kv[e] * (eGp * sc[3]);
            } else {
                Rt[e] = rv[e] * eG;
                Bt[e] = bv[e] * eGp;
                Ah[e] = av[e] * enG;
                Kh[e] = kv[e] * enG;
            }
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

        op.B[s] = Bh;
        // Gated DeltaNet: R~ = (e^{G_t} / |q_t|) q_t with q_t exact in bf16, so the
        // consumer multiplies q_t S instead and scales the result by op.sig.
        if constexpr (GDN)
            op.R[s] = __builtin_bit_cast(bf16x8, u32x4{rt.x[s][0][0][0], rt.x[s][0][0][1], rt.x[s][0][1][0],
                                                       rt.x[s][0][1][1]});
        else
            op.R[s] = Rh;
        op.ah[s] = __builtin_bit_cast(u32x4, Ahh);
        op.kh[s] = __builtin_bit_cast(u32x4, Khh);
        op.kl[s] = __builtin_bit_cast(u32x4, Khl);
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
    op.tinv = cvt4(mfma16(cvt4(t4), n8t, t4t));
    op.tnbk = cvt4(mfma16(cvt4(mbk), op.tinv, zero4()));
    op.mra = cvt4(mraT);
    split4(mrkT, op.mrkh, op.mrkl);
    op.flag = __any((int)(emin < kMinChunkFactor || wmax[0] > 0 || wmax[1] > 0)) ? 1 : 0;
}

// Producer: write one chunk's operands into `slot` (layout WS<D>).
template <int D, bool GDN>
__device__ __forceinline__ void ws_store_ops(const ChunkOps<D> &op, char *slot, int lane)
{
    using C = WS<D>;
    const int t = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < C::NCB; ++s) {
        st16(slot + C::OFF_B + s * 1024 + lane * 16, op.B[s]);
        st16(slot + C::OFF_R + s * 1024 + lane * 16, op.R[s]);
        // Row t of the A^, K^ hi and K^ lo tiles, channels 32s + 16hh + 4g .. +3.
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int off = tile_off<D>(t, 32 * s + 16 * hh + 4 * g);
            *(u32x2 *)(slot + C::OFF_AH + off) = u32x2{op.ah[s][2 * hh], op.ah[s][2 * hh + 1]};
            *(u32x2 *)(slot + C::OFF_KH + off) = u32x2{op.kh[s][2 * hh], op.kh[s][2 * hh + 1]};
            *(u32x2 *)(slot + C::OFF_KL + off) = u32x2{op.kl[s][2 * hh], op.kl[s][2 * hh + 1]};
        }
        // e^{G_L} (one writer per row)
        if (t == 0) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                *(f32x4 *)(slot + C::OFF_EGL + (32 * s + 16 * hh + 4 * g) * 4) = op.egl[s][hh];
        }
    }
    st8(slot + C::OFF_TN + lane * 16, op.tinv);
    st8(slot + C::OFF_TN + lane * 16 + 8, op.tnbk);
    st8(slot + C::OFF_MM + lane * 16, op.mra);
    st8(slot + C::OFF_MM + lane * 16 + 8, op.mrkh);
    st8(slot + C::OFF_MRKL + lane * 8, op.mrkl);
    if constexpr (GDN) {
        if (g == 0) *(float *)(slot + C::OFF_SIG + 4 * t) = op.sig;
    }
}

// ---- consumer ----------------------------------------------------------------
//
// S[q][n] holds rows 16q + 4g + i, column cbase + 16n + j of the state (lane
// (g = l/16, j = l%16)), n < NT; cbase = CW x the consumer's index.

// Exact path: token-by-token fp32 update of the consumer's column slice.
template <int D>
__device__ void ws_chunk_exact(f32x4 (*S)[WS<D>::NT], const uint16_t *r, const uint16_t *w,
                               const uint16_t *k, const uint16_t *v, const uint16_t *a,
                               const uint16_t *b, const uint8_t *mask, uint16_t *o, size_t tok0, int Tn,
                               int H, int h, int chunk, int cbase, int lane)
{
    constexpr int NQ = D / 16, NT = WS<D>::NT;
    const int g = lane >> 4, j = lane & 15;
    for (int tt = 0; tt < 16; ++tt) {
        const int tok = chunk * 16 + tt;
        if (tok >= Tn) break;
        const bool upd = mask == nullptr || mask[tok0 + tok] != 0;
        const size_t base = ((tok0 + tok) * H + h) * D;
        if (upd) {
            float sb[NT] = {};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if constexpr (NQ > 4) __builtin_amdgcn_sched_barrier(0);   // bound the hoisted loads
                const u32x2 bq = *(const u32x2 *)(b + base + 16 * q + 4 * g);
                const float be[4] = {bf16_lo(bq[0]), bf16_hi(bq[0]), bf16_lo(bq[1]), bf16_hi(bq[1])};
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sb[n] = fmaf(be[i], S[q][n][i], sb[n]);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) sb[n] = xsum32(xsum16(sb[n]));
            float vj[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) vj[n] = bf16_bits_to_f32(v[base + cbase + 16 * n + j]);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if constexpr (NQ > 4) __builtin_amdgcn_sched_barrier(0);
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
                    for (int n = 0; n < NT; ++n)
                        S[q][n][i] = fmaf(d, S[q][n][i], fmaf(ae[i], sb[n], ke[i] * vj[n]));
                }
            }
        }
        float ov[NT] = {};
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if constexpr (NQ > 4) __builtin_amdgcn_sched_barrier(0);
            const u32x2 rq = *(const u32x2 *)(r + base + 16 * q + 4 * g);
            const float re[4] = {bf16_lo(rq[0]), bf16_hi(rq[0]), bf16_lo(rq[1]), bf16_hi(rq[1])};
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[n] = fmaf(re[i], S[q][n][i], ov[n]);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) ov[n] = xsum32(xsum16(ov[n]));
        if (g == 0) {
#pragma unroll
            for (int n = 0; n < NT; ++n) o[base + cbase + 16 * n + j] = f32_to_bf16_bits(ov[n]);
        }
    }
}

// Exact path, Gated DeltaNet inputs (q, k, v, per-token gate g and strength
// beta); same state layout as ws_chunk_exact.
template <int D>
__device__ void ws_chunk_exact_gdn(f32x4 (*S)[WS<D>::NT], const uint16_t *q, const uint16_t *gg,
                                   const uint16_t *k, const uint16_t *v, const uint16_t *beta,
                                   uint16_t *o, size_t tok0, int Tn, int H, int h, int chunk, int cbase,
                                   int lane)
{
    constexpr int NQ = D / 16, NT = WS<D>::NT;
    const int g = lane >> 4, j = lane & 15;
    auto ld4 = [&](const uint16_t *p, float *x) {
        const u32x2 u = *(const u32x2 *)p;
        x[0] = bf16_lo(u[0]); x[1] = bf16_hi(u[0]); x[2] = bf16_lo(u[1]); x[3] = bf16_hi(u[1]);
    };
    for (int tt = 0; tt < 16; ++tt) {
        const int tok = chunk * 16 + tt;
        if (tok >= Tn) break;
        const size_t sidx = (tok0 + tok) * H + h;
        const size_t base = sidx * D;
        const float gate = bf16_bits_to_f32(gg[sidx]), bt = bf16_bits_to_f32(beta[sidx]);
        // Norms (lanes of one row group hold the same channels: reduce over
        // the groups only), then k^T S; q and k are re-read where used so
        // that this rare path keeps few registers live.
        float nq = 0.0f, nk = 0.0f;
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if constexpr (NQ > 4) __builtin_amdgcn_sched_barrier(0);
            float qe[4], ke[4];
            ld4(q + base + 16 * qi + 4 * g, qe);
            ld4(k + base + 16 * qi + 4 * g, ke);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                nq = fmaf(qe[i], qe[i], nq);
                nk = fmaf(ke[i], ke[i], nk);
            }
        }
        nq = xsum32(xsum16(nq));
        nk = xsum32(xsum16(nk));
        const float iq = 1.0f / sqrtf(nq + 1e-6f), ik = 1.0f / sqrtf(nk + 1e-6f);
        const float alpha = __expf(gate);
        float ks[NT] = {};
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if constexpr (NQ > 4) __builtin_amdgcn_sched_barrier(0);
            float ke[4];
            ld4(k + base + 16 * qi + 4 * g, ke);
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) ks[n] = fmaf(ke[i] * ik, S[qi][n][i], ks[n]);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) ks[n] = xsum32(xsum16(ks[n]));
        float vj[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) vj[n] = bf16_bits_to_f32(v[base + cbase + 16 * n + j]);
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if constexpr (NQ > 4) __builtin_amdgcn_sched_barrier(0);
            float ke[4];
            ld4(k + base + 16 * qi + 4 * g, ke);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float kn = ke[i] * ik;
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    S[qi][n][i] = fmaf(alpha, fmaf(-bt * kn, ks[n], S[qi][n][i]), bt * kn * vj[n]);
            }
        }
        float ov[NT] = {};
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if constexpr (NQ > 4) __builtin_amdgcn_sched_barrier(0);
            float qe[4];
            ld4(q + base + 16 * qi + 4 * g, qe);
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) ov[n] = fmaf(qe[i] * iq, S[qi][n][i], ov[n]);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) ov[n] = xsum32(xsum16(ov[n]));
        if (g == 0) {
#pragma unroll
            for (int n = 0; n < NT; ++n) o[base + cbase + 16 * n + j] = f32_to_bf16_bits(ov[n]);
        }
    }
}

// Store one chunk's output tile held as O^T fragments (lane (g, t): token t,
// columns cbase + 16n + 4g .. +3).
template <int D>
__device__ __forceinline__ void ws_store_out(const f32x4 *Ot, uint16_t *o, size_t tok0, int Tn, int H,
                                             int h, int chunk, int cbase, int lane)
{
    const int g = lane >> 4, t = lane & 15;
    const int tok = chunk * 16 + t;
    if (tok < Tn) {
        uint16_t *op = o + ((tok0 + tok) * H + h) * D + cbase + 4 * g;
#pragma unroll
        for (int n = 0; n < WS<D>::NT; ++n)
            *(u32x2 *)(op + 16 * n) = u32x2{cvt2_bits(Ot[n][0], Ot[n][1]), cvt2_bits(Ot[n][2], Ot[n][3])};
    }
}

// The S-dependent part of one chunk for the consumer's 64 columns.  Work is
// issued in dependency order across the four independent column tiles, and
// the S-independent products are placed where they fill the latency of the
// S -> X -> U -> S' chain.
template <int D, bool GDN>
__device__ __forceinline__ void ws_chunk_serial(f32x4 (*S)[WS<D>::NT], const char *slot, uint16_t *o,
                                                size_t tok0, int Tn, int H, int h, int chunk, int cbase,
                                                int lane)
{
    using C = WS<D>;
    constexpr int NT = C::NT;
    const int g = lane >> 4;
    // bf16 copy of the chunk-start state as MFMA fragments: block s pairs row
    // tiles 2s and 2s + 1 (k-slot 4hh + i of lane group g is channel
    // 32s + 16hh + 4g + i, the producer's channel order).
    bf16x8 sb[C::NCB][NT];
    bf16x4 vf[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int s = 0; s < C::NCB; ++s) sb[s][n] = cat8(cvt4(S[2 * s][n]), cvt4(S[2 * s + 1][n]));
        vf[n] = tile_tr<D>(slot + C::OFF_V, 4 * g, cbase + 16 * n, lane);   // V[4g + i][cbase + 16n + j]
    }
    f32x4 Ot[NT];   // O^T
    if constexpr (GDN) {
        // Gated DeltaNet: the S-part of the output is (e^{G_t} / |q_t|) q_t S
        // with q_t exact; q_t S is taken to about 16 bits by adding the bf16
        // state's remainder as a second term (computed here, before S
        // changes).  On random q this output term is a small projection of a
        // larger state, and a bf16 state alone costs most of the error budget.
#pragma unroll
        for (int s = 0; s < C::NCB; ++s) {
            const bf16x8 rt = ld16(slot + C::OFF_R + s * 1024 + lane * 16);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                f32x4 l0 = S[2 * s][n], l1 = S[2 * s + 1][n];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    l0[i] -= (float)sb[s][n][i];
                    l1[i] -= (float)sb[s][n][4 + i];
                }
                Ot[n] = mfma32(cat8(cvt4(l0), cvt4(l1)), rt, s == 0 ? zero4() : Ot[n]);
            }
        }
    }
    // X = B~ S
    f32x4 X[NT];
    {
        const bf16x8 bt = ld16(slot + C::OFF_B + lane * 16);
#pragma unroll
        for (int n = 0; n < NT; ++n) X[n] = mfma32(bt, sb[0][n], zero4());
    }
    // S += K^lo^T V  (independent of X; the decay is applied at the end)
#pragma unroll
    for (int q = 0; q < C::NQ; ++q) {
        const bf16x4 ktl = tile_tr<D>(slot + C::OFF_KL, 4 * g, 16 * q, lane);
#pragma unroll
        for (int n = 0; n < NT; ++n) S[q][n] = mfma16(ktl, vf[n], S[q][n]);
    }
#pragma unroll
    for (int s = 1; s < C::NCB; ++s) {
        const bf16x8 bt = ld16(slot + C::OFF_B + s * 1024 + lane * 16);
#pragma unroll
        for (int n = 0; n < NT; ++n) X[n] = mfma32(bt, sb[s][n], X[n]);
    }
    // O^T, S-part (chunk-start state)
#pragma unroll
    for (int s = 0; s < C::NCB; ++s) {
        const bf16x8 rt = ld16(slot + C::OFF_R + s * 1024 + lane * 16);
#pragma unroll
        for (int n = 0; n < NT; ++n) Ot[n] = mfma32(sb[s][n], rt, (s == 0 && !GDN) ? zero4() : Ot[n]);
    }
    if constexpr (GDN) {
        const float sig = *(const float *)(slot + C::OFF_SIG + 4 * (lane & 15));
#pragma unroll
        for (int n = 0; n < NT; ++n) Ot[n] *= sig;
    }
    // U = T X + N_bk V
    const bf16x8 tn = ld16(slot + C::OFF_TN + lane * 16);
    bf16x8 uv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) uv[n] = cat8(cvt4(mfma32(tn, cat8(cvt4(X[n]), vf[n]), zero4())), vf[n]);
    const bf16x4 mrkl = ld8(slot + C::OFF_MRKL + lane * 8);
#pragma unroll
    for (int n = 0; n < NT; ++n) Ot[n] = mfma16(vf[n], mrkl, Ot[n]);
    // S <- diag(e^{G_L}) (S + [A^^T | K^hi^T] [U; V])
#pragma unroll
    for (int q = 0; q < C::NQ; ++q) {
        // At D = 128 the operand reads of the 8 row tiles are not all hoisted
        // to the top (that would not fit in the register file).
        if constexpr (C::NQ > 4) {
            if (q % 4 == 0) __builtin_amdgcn_sched_barrier(0);
        }
        const bf16x8 atk = cat8(tile_tr<D>(slot + C::OFF_AH, 4 * g, 16 * q, lane),
                                tile_tr<D>(slot + C::OFF_KH, 4 * g, 16 * q, lane));
        const f32x4 eg = *(const f32x4 *)(slot + C::OFF_EGL + (16 * q + 4 * g) * 4);
#pragma unroll
        for (int n = 0; n < NT; ++n) S[q][n] = mfma32(atk, uv[n], S[q][n]) * eg;
    }
    // O^T += [U; V]^T [M_ra | M_rk]^T
    const bf16x8 mm = ld16(slot + C::OFF_MM + lane * 16);
#pragma unroll
    for (int n = 0; n < NT; ++n) Ot[n] = mfma32(uv[n], mm, Ot[n]);
    ws_store_out<D>(Ot, o, tok0, Tn, H, h, chunk, cbase, lane);
}

// ---- kernel --------------------------------------------------------------------

// GDN = false: generalized-delta-rule inputs r, w, k, v, a, b.  GDN = true:
// Gated DeltaNet inputs in the same argument slots: r = q, k = k, v = v,
// w = g [.., H], a = beta [.., H] (b and mask unused).
template <int D, bool GDN, bool ORDERED>
__global__ __launch_bounds__(64 * WS<D>::NWAVE)
__attribute__((amdgpu_waves_per_eu(WS<D>::WAVES_PER_SIMD, WS<D>::WAVES_PER_SIMD))) void chunked_ws_kernel(
    int T, int H, int nbh, const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ state_map,
    int n_state, const uint16_t *__restrict__ r, const uint16_t *__restrict__ w,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const uint16_t *__restrict__ a,
    const uint16_t *__restrict__ b, const float *__restrict__ s0, const uint8_t *__restrict__ mask,
    uint16_t *__restrict__ o, float *__restrict__ sf, int wait_limit)
{
    using C = WS<D>;
    // Separate LDS objects: the compiler must wait for outstanding
    // global->LDS loads before touching the object they write (the raw
    // buffers), but not before the slot rings or the hand-off counters.
    __shared__ __attribute__((aligned(256))) char lds_slots[C::LDS_SLOTS];
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_RAW];
    __shared__ int lds_sync[32];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int g = lane >> 4, j = lane & 15;
    constexpr int NC = C::NSEQ * C::NCONS;   // consumers per workgroup

    // Role assignment by SIMD placement.  The consumers (mostly MFMA work,
    // slowed down by sharing a SIMD with VALU-heavy producers) are taken
    // from the SIMDs with the fewest workgroup waves, at most one per SIMD
    // while that is possible.  The other waves become producers, alternating
    // between the sequences in (SIMD, wave) order so that each sequence's
    // producers are spread over different SIMDs.  (Measured at D = 64: eight
    // waves with three producers per sequence beat six waves with two, where
    // the consumers run alone on a SIMD but production falls behind.)
    // Correctness does not depend on the placement; it only picks which wave
    // does what (every placement yields each role exactly once).
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
    const bool is_cons = crank < NC;
#pragma unroll
    for (int w2 = 0; w2 < C::NWAVE; ++w2) {
        int cr = 0;
#pragma unroll
        for (int w3 = 0; w3 < C::NWAVE; ++w3) cr += ckey[w3] < ckey[w2] ? 1 : 0;
        prank += (cr >= NC && key_of[w2] < key_of[wave]) ? 1 : 0;
    }
    const int seq = is_cons ? crank % C::NSEQ : prank % C::NSEQ;
    // Workgroups go to the eight XCDs round robin (workgroup i to XCD i % 8).
    // With sequences of one length and a grid that divides evenly, each XCD
    // takes a contiguous range of sequences, so that the heads of one token
    // share an XCD and its L2 fetches the values every head of the token
    // reads (the mask; the gate and strength of Gated DeltaNet) once: Gated
    // DeltaNet's fetch fell from 1.073x to 1.0004x the algorithmic bytes.
    // Packed sequences of mixed lengths keep the round robin, which spreads
    // a long sequence's heads over all XCDs (contiguous ranges measured
    // 0.490 against 0.470 ms on the packed benchmark batch).
    const unsigned nwg = gridDim.x;
    const unsigned wg = (!cu_seqlens && nwg % 8u == 0u) ? (blockIdx.x % 8u) * (nwg / 8u) + blockIdx.x / 8u
                                                        : blockIdx.x;
    const int bh = (int)wg * C::NSEQ + seq;
    // Packed calls with few sequences take them longest first: rank bh / H
    // of the workgroup order is the sequence of that rank by length, so the
    // longest chains start in the first dispatch round instead of running
    // alone at the end when drawn late (the whole workgroup, before any wave
    // leaves).
    // ORDERED (chosen on the host, use_longest_first) compiles this in;
    // the other calls keep the plain order.
    int sq_ranked = -1, lf_tb = 0, lf_tn = 0;
    if constexpr (ORDERED) {
        __shared__ int lf_beg[kLongestFirstMax], lf_len[kLongestFirstMax], lf_rank[kLongestFirstMax],
            lf_pick[C::NSEQ];
        longest_first<C::NSEQ>(cu_seqlens, T, nbh / H, (int)wg * C::NSEQ, H, lf_beg, lf_len, lf_rank, lf_pick);
        sq_ranked = lf_pick[seq];
        if (sq_ranked >= 0) {
            lf_tb = lf_beg[sq_ranked];
            lf_tn = lf_len[sq_ranked];
        }
    }
    if (bh >= nbh) return;
    // Sequence sq: tokens [tok0, tok0 + Tn) of the (packed) token axis,
    // initial state row sidx of the state pool (-1: zeros).  Offsets and
    // state indices read from device memory are clamped into range.
    const int h = bh % H, sq = ORDERED ? sq_ranked : bh / H;
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
    const int nchunks = (Tn + 15) / 16;
    char *const lds = lds_slots + seq * C::NSLOT * C::SLOT;
    // Per sequence: ready[NSLOT], then one done counter per consumer (a sum
    // over consumers would let a consumer running ahead release a slot that
    // a slower one is still reading).
    // The eighth counter is the sequence's failure flag: set when a producer
    // gave up waiting for a slot and overwrote it while it may still be read.
    int *ready = lds_sync + 8 * seq;
    int *done = ready + C::NSLOT;
    int *failed = ready + 7;
    static_assert(C::NSLOT + C::NCONS <= 7, "hand-off counters of one sequence");

    if (is_cons) {
        // ---------------- consumer: columns cbase .. cbase + CW - 1 ----------------
        const int cbase = C::CW * (crank / C::NSEQ);
        f32x4 S[C::NQ][C::NT];
        const size_t st_base = (size_t)(ORDERED ? sq * H + h : bh) * D * D;   // final state [N, H, D, D]
        const size_t st_in = ((size_t)(sidx < 0 ? 0 : sidx) * H + h) * D * D;   // initial state pool
#pragma unroll
        for (int q = 0; q < C::NQ; ++q)
#pragma unroll
            for (int n = 0; n < C::NT; ++n) S[q][n] = zero4();
        if (s0 && sidx >= 0) {
#pragma unroll
            for (int q = 0; q < C::NQ; ++q)
#pragma unroll
                for (int n = 0; n < C::NT; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[q][n][i] = s0[st_in + (size_t)(16 * q + 4 * g + i) * D + cbase + 16 * n + j];
        }
        // With the Gated DeltaNet inputs and at D = 128 the initial state is
        // made complete before the chunk loop.  Otherwise the state registers
        // count as loads in flight at the loop head, and every chunk's first
        // reads of the state wait for all memory operations in flight, the
        // previous chunk's output stores included.  Measured: Gated DeltaNet
        // d64 0.381 -> 0.371 ms, WKV7 d128 about 1 % faster; the WKV7 d64
        // path keeps the wait (0.400 -> 0.424 ms without it: its consumers
        // then run ahead, and its producers, heavier than the Gated DeltaNet
        // ones, wait longer for the value tile).
        if constexpr (GDN || D == 128) {
#pragma unroll
            for (int q = 0; q < C::NQ; ++q)
#pragma unroll
                for (int n = 0; n < C::NT; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(S[q][n][i]));
        }
        // A hand-off that gave up poisons the results: the state becomes NaN
        // (so every later output and the final state are NaN), and so do the
        // output rows of a chunk that may have been read from a slot in an
        // unknown state.  A producer sets the failure flag before it
        // overwrites a slot that may still be read, so a consumer whose slot
        // reads for chunk c returned overwritten data sees the flag at its
        // next poll (the wait for chunk c + 1, or the check after the loop):
        // the chunk to poison is then the previous one.
        bool poisoned = false;
        auto poison = [&](int c_out) {
#pragma unroll
            for (int q = 0; q < C::NQ; ++q)
#pragma unroll
                for (int n = 0; n < C::NT; ++n) S[q][n] = f32x4{NAN, NAN, NAN, NAN};
            if (c_out >= 0) {
                f32x4 Ot[C::NT];
#pragma unroll
                for (int n = 0; n < C::NT; ++n) Ot[n] = f32x4{NAN, NAN, NAN, NAN};
                ws_store_out<D>(Ot, o, tok0, Tn, H, h, c_out, cbase, lane);
            }
            poisoned = true;
        };
        for (int c = 0; c < nchunks; ++c) {
            const char *slot = lds + (c % C::NSLOT) * C::SLOT;
            // ready[slot] = 2 (c + 1) + extreme-decay flag once chunk c is in the slot
            int fail_seen;
            const int rv = spin_ge(&ready[c % C::NSLOT], 2 * (c + 1), wait_limit, failed, fail_seen);
            const bool gave_up = rv < 2 * (c + 1);
            if (__builtin_expect(gave_up || (fail_seen && !poisoned), 0)) {
                if (gave_up) lds_store_relaxed(failed, 1);
                // S = NaN, so this chunk's outputs come out NaN; a flag seen
                // for the first time also poisons the previous chunk
                poison(fail_seen && !poisoned ? c - 1 : -1);
            }
            if (!gave_up && (rv & 1)) {
                if constexpr (GDN)
                    ws_chunk_exact_gdn<D>(S, r, w, k, v, a, o, tok0, Tn, H, h, c, cbase, lane);
                else
                    ws_chunk_exact<D>(S, r, w, k, v, a, b, mask, o, tok0, Tn, H, h, c, cbase, lane);
            } else
                ws_chunk_serial<D, GDN>(S, slot, o, tok0, Tn, H, h, c, cbase, lane);
            lds_wait();                          // all reads of the slot have returned
            lds_store_relaxed(&done[crank / C::NSEQ], c + 1);
        }
        if (nchunks > 0 && !poisoned && lds_load_relaxed(failed)) poison(nchunks - 1);
        if (sf) {
#pragma unroll
            for (int q = 0; q < C::NQ; ++q)
#pragma unroll
                for (int n = 0; n < C::NT; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sf[st_base + (size_t)(16 * q + 4 * g + i) * D + cbase + 16 * n + j] = S[q][n][i];
        }
    } else {
        // ---------------- producers ----------------
        const int p = prank / C::NSEQ;
        char *raw = lds_raw + (seq * C::NPROD + p) * C::RAW;
        const uint32_t raw_lds = lds_addr(raw);
        // Element offset of (bb, token 0, h, channel 0) and between tokens.
        const size_t seq_base = (tok0 * H + h) * D;
        const uint32_t tok_stride = (uint32_t)H * D;
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
        // Loop-carried requests for this producer's next chunk: the mask byte
        // (or, for Gated DeltaNet, the gate and strength) of token
        // (next chunk, lane & 15).
        uint32_t mnext = 1, gnext = 0, bnext = 0;
        const int t = lane & 15;
        if (p < nchunks) {
            ws_issue_raw<D, GDN>(raw_lds, src, seq_base, tok_stride, Tn, p, lane);
            const size_t tk = tok0 + min(p * 16 + t, Tn - 1);
            if constexpr (GDN) {
                gnext = w[tk * H + h];
                bnext = a[tk * H + h];
            } else {
                if (mask) mnext = mask[tk];
            }
        }
        for (int c = p; c < nchunks; c += C::NPROD) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            const uint32_t mcur = mnext, gcur = gnext, bcur = bnext;
            RawTile<D> rt;
            ws_read_raw<D, GDN>(rt, raw, lane);
            lds_wait();
            if (c + C::NPROD < nchunks) {
                const int cn = c + C::NPROD;
                ws_issue_raw<D, GDN>(raw_lds, src, seq_base, tok_stride, Tn, cn, lane);
                const size_t tk = tok0 + min(cn * 16 + t, Tn - 1);
                if constexpr (GDN) {
                    gnext = w[tk * H + h];
                    bnext = a[tk * H + h];
                } else {
                    if (mask) mnext = mask[tk];
                }
            }
            float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (GDN) gdn_scalars<D>(rt, gcur, bf16_bits_to_f32((uint16_t)bcur), sc);
            const int tok = c * 16 + t;
            rt.valid = tok < Tn;
            rt.upd = rt.valid && mcur != 0;
            zero_inactive<D>(rt);
            const bool all_upd = __all(rt.upd);
            ChunkOps<D> op;
            ws_precompute<D, GDN>(rt, op, lane, psel, ltri, sc);
            char *slot = lds + (c % C::NSLOT) * C::SLOT;
            // the slot's previous chunk is consumed by every consumer
            if (!spin_all_ge<C::NCONS>(done, c - C::NSLOT + 1, wait_limit)) {
                lds_store_relaxed(failed, 1);
                lds_wait();                      // flag set before the slot is overwritten
            }
            ws_issue_v<D>(lds_addr(slot + C::OFF_V), v, seq_base, tok_stride, Tn, c, lane);
            ws_store_ops<D, GDN>(op, slot, lane);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the value tile has landed
            if (!all_upd && !rt.upd) {
                // Value rows of tokens that do not update are cleared, so that
                // whatever they hold (even inf or nan) cannot reach the state.
                const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int cc = 0; cc < D / 32; ++cc)
                    *(u32x4 *)(slot + C::OFF_V + tile_off<D>(t, (D / 4) * g + 8 * cc)) = zero;
            }
            lds_wait();
            lds_store_relaxed(&ready[c % C::NSLOT], 2 * (c + 1) + op.flag);
        }
    }
}

template <int D, bool GDN, bool ORDERED>
static hipError_t launch_ws(const FwdArgs &p, hipStream_t stream)
{
    using C = WS<D>;
    const int nbh = p.B * p.H;
    const dim3 grid((unsigned)((nbh + C::NSEQ - 1) / C::NSEQ)), block(64 * C::NWAVE);
    hipLaunchKernelGGL((chunked_ws_kernel<D, GDN, ORDERED>), grid, block, 0, stream, p.T, p.H, nbh, p.cu_seqlens,
                       p.state_map, p.n_state,
                       (const uint16_t *)p.r, (const uint16_t *)p.w, (const uint16_t *)p.k,
                       (const uint16_t *)p.v, (const uint16_t *)p.a, (const uint16_t *)p.b, p.s0,
                       p.mask, (uint16_t *)p.o, p.sf, current_wait_limit());
    return hipGetLastError();
}

hipError_t launch_chunked(const FwdArgs &p, hipStream_t stream)
{
    // packed calls of few, long enough sequences take them longest first
    if (use_longest_first(p.cu_seqlens != nullptr, p.B, p.T)) {
        if (p.gdn) return p.D == 64 ? launch_ws<64, true, true>(p, stream) : launch_ws<128, true, true>(p, stream);
        return p.D == 64 ? launch_ws<64, false, true>(p, stream) : launch_ws<128, false, true>(p, stream);
    }
    if (p.gdn) return p.D == 64 ? launch_ws<64, true, false>(p, stream) : launch_ws<128, true, false>(p, stream);
    return p.D == 64 ? launch_ws<64, false, false>(p, stream) : launch_ws<128, false, false>(p, stream);
}

}  // namespace wkv7

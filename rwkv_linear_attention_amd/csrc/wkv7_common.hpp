// Device helpers shared by the WKV7 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- bf16 <-> fp32 -------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }

// Round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 cvt2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_convertvector(v, bf16x2);
}
__device__ __forceinline__ uint32_t cvt2_bits(float a, float b) {
    bf16x2 p = cvt2(a, b);
    return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float a) {
    return (uint16_t)(cvt2_bits(a, 0.0f) & 0xffffu);
}
// Written as two pair conversions: a whole-vector conversion can be lowered
// to one conversion per element plus byte permutes.
__device__ __forceinline__ bf16x4 cvt4(f32x4 v) {
    const u32x2 p = {cvt2_bits(v[0], v[1]), cvt2_bits(v[2], v[3])};
    return __builtin_bit_cast(bf16x4, p);
}

// Element loaders for the two I/O types.  bf16 travels as raw uint16_t.
template <typename T> struct io;
template <> struct io<float> {
    __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float *p, size_t i, float x) { p[i] = x; }
};
template <> struct io<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t *p, size_t i) { return bf16_bits_to_f32(p[i]); }
    __device__ __forceinline__ static void store(uint16_t *p, size_t i, float x) { p[i] = f32_to_bf16_bits(x); }
};

// Four consecutive elements kept in their I/O type (a prefetch register set).
template <typename T> struct raw4;
template <> struct raw4<float> {
    typedef f32x4 type;
    __device__ __forceinline__ static type load(const float *p, size_t i) { return *(const f32x4 *)(p + i); }
    __device__ __forceinline__ static f32x4 f32(type x) { return x; }
    __device__ __forceinline__ static type zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
};
template <> struct raw4<uint16_t> {
    typedef u32x2 type;
    __device__ __forceinline__ static type load(const uint16_t *p, size_t i) { return *(const u32x2 *)(p + i); }
    __device__ __forceinline__ static f32x4 f32(type u)
    {
        return f32x4{bf16_lo(u[0]), bf16_hi(u[0]), bf16_lo(u[1]), bf16_hi(u[1])};
    }
    __device__ __forceinline__ static type zero() { return u32x2{0u, 0u}; }
};
// ---- cross-lane ----------------------------------------------------------

// row_shr:n inside each 16-lane row; lanes without a source receive `fill`.
template <int N>
__device__ __forceinline__ float row_shr(float x, float fill) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x),
                                                      0x110 + N, 0xF, 0xF, false));
}
// Broadcast lane 15 of each 16-lane row to the whole row (row_newbcast:15).
__device__ __forceinline__ float row_bcast15(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x15F, 0xF, 0xF, false));
}
// Inclusive prefix sum over the 16 lanes of each row (Hillis-Steele).
__device__ __forceinline__ float row_scan16(float x) {
    x += row_shr<1>(x, 0.0f);
    x += row_shr<2>(x, 0.0f);
    x += row_shr<4>(x, 0.0f);
    x += row_shr<8>(x, 0.0f);
    return x;
}

__device__ __forceinline__ float xor_sum(float x, int mask) { return x + __shfl_xor(x, mask, kWave); }

// x plus its value in the lane 16 (32) apart, with gfx950's lane-swap VALU
// instructions instead of an LDS permute: permlane16_swap exchanges the odd
// 16-lane rows of one operand with the even rows of the other, so with x in
// both operands the two results hold x and its partner (in some order) in
// every lane; permlane32_swap does the same for the two 32-lane halves.
// Addition is commutative, so the sums equal x + shfl_xor(x, 16 / 32) bit
// for bit.
__device__ __forceinline__ float xsum16(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xsum32(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Gated DeltaNet operands.  With kn = k / sqrt(|k|^2 + 1e-6) (qn likewise),
// the gated delta rule S = e^g (I - beta kn kn^T) S + beta kn v^T, o = S^T qn
// (rwkv-ops README, section "gdn_recurrent 使用方法", read as the textbook rule)
// is the generalized rule with r = qn, w = g on every channel, k = beta kn,
// a = -e^g beta kn and b = kn.  The staging steps below form those operands
// from q, k, g and beta, one thread per four channels of a token; the D/4
// threads of a token are adjacent lanes of one wave.
constexpr float kGdnNormEps = 1e-6f;

// Sum over the D/4 lanes of a token with DPP (no LDS traffic): swap lane
// pairs, then pairs of pairs, then mirror within each 8- and 16-lane half
// (row_half_mirror, row_mirror); at D = 128 also add the neighbouring 16-lane
// row.  Each step adds two partial sums in either order, so every lane of the
// token ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int D>
__device__ __forceinline__ float token_sum(float x)
{
    static_assert(D == 64 || D == 128, "a token spans 16 or 32 lanes");
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);   // row_half_mirror
    x += dpp_mov<0x140>(x);   // row_mirror
    if constexpr (D == 128) x = xsum16(x);
    return x;
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

// 1 / sqrt(|x|^2 + eps) over the whole token row (x: this thread's 4 channels).
template <int D>
__device__ __forceinline__ float inv_norm(f32x4 x)
{
    return 1.0f / sqrtf(token_sum<D>(dot4(x, x)) + kGdnNormEps);
}

// ---- MFMA ----------------------------------------------------------------
// 16x16x32 bf16: lane l supplies A[m = l%16][8 k-slots of group l/16] and
// B[8 k-slots of group l/16][n = l%16]; the accumulator holds
// D[4*(l/16) + i][l%16], i = 0..3.  16x16x16 is the same with 4 k-slots.

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Wave-local LDS ordering: all LDS traffic issued so far has completed.
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// ---- packed sequences ------------------------------------------------------
// Longest-first order of packed sequences (at most kLongestFirstMax of them,
// so that every workgroup can rank them all in LDS at its start).  Workgroups
// are dispatched in index order; taking the longest sequences first keeps a
// long sequence drawn late from running alone at the end.  The rank of
// sequence i is the number of sequences longer than it, or as long with a
// smaller index: a permutation of 0 .. nseq - 1.  pick[s] becomes the
// sequence of rank (bh0 + s) / H, the s-th (sequence, head) slot of this
// workgroup; slots past the last sequence keep -1.  beg[i] and len[i] hold
// sequence i's first token and length, clamped as the kernels clamp them.
// The threads split the comparisons (kLongestFirstMax sequences times
// blockDim.x / kLongestFirstMax slices of the others) and add their counts
// into rank[] in LDS.  Every thread of the workgroup calls it (three
// barriers); blockDim.x is a multiple of kLongestFirstMax.
constexpr int kLongestFirstMax = 128;

// Packed calls that take the longest-first order: at most kLongestFirstMax
// sequences, averaging at least 256 tokens.  The ranking costs about a
// microsecond at each workgroup's start; 128 sequences of 16 tokens measured
// 148 against 129 us without it, of 64 tokens 240 against 224 us, of 256
// tokens 501 against 505 us.
__host__ __device__ constexpr bool use_longest_first(bool packed, long long nseq, long long total_T)
{
    return packed && nseq <= kLongestFirstMax && total_T >= 256 * nseq;
}

template <int NSEQ>
__device__ __forceinline__ void longest_first(const int32_t *cu, int T, int nseq, int bh0, int H, int *beg,
                                              int *len, int *rank, int *pick)
{
    const int tid = threadIdx.x, nt = blockDim.x;
    if (tid < nseq) {
        const int tb = min(max(cu[tid], 0), T);
        beg[tid] = tb;
        len[tid] = min(max(cu[tid + 1], tb), T) - tb;
        rank[tid] = 0;
    }
    if (tid < NSEQ) pick[tid] = -1;
    __syncthreads();
    const int parts = nt / kLongestFirstMax;
    const int i = tid % kLongestFirstMax, part = tid / kLongestFirstMax;
    if (i < nseq) {
        const int span = (nseq + parts - 1) / parts, j0 = part * span, j1 = min(j0 + span, nseq);
        const int li = len[i];
        int r = 0;
#pragma unroll 8
        for (int j = j0; j < j1; ++j) {
            const int lj = len[j];
            r += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        if (r) atomicAdd(&rank[i], r);
    }
    __syncthreads();
    if (tid < nseq) {
        const int r = rank[tid];
#pragma unroll
        for (int sl = 0; sl < NSEQ; ++sl)
            if (r == (bh0 + sl) / H) pick[sl] = tid;
    }
    __syncthreads();
}

}  // namespace wkv7

// C ABI of libwkv7.so: argument validation, path choice and launches.
// Declarations and the contract of every entry point: include/wkv7.h.
#include <stdint.h>

#include <atomic>

#include "../../include/wkv7.h"
#include "wkv7_common.hpp"
#include "wkv7_internal.hpp"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Sequences shorter than this run on the recurrent kernel under AUTO.
// Measured on MI355X (bf16, head size 64 and 128, 1 to 512 sequences): from
// T = 16 on the chunked kernel is as fast or faster for every shape (equal
// within call overhead for small batches at T = 16, up to 1.6x faster there
// with 512 sequences; 4.7x to 8.9x at T = 2048).  Below 16 the two are within
// call overhead except at head size 128 with 512 sequences, where the
// recurrent kernel is faster at T <= 4 (12-16 vs 21 us) and slower at T = 8
// (22.6 vs 20.9 us).
constexpr int kChunkedMinT = 16;
// fp32 I/O (WKV7; Gated DeltaNet fp32 runs on the recurrent kernel): the
// same threshold, measured the same way.  From T = 16 the fp32 chunked kernel
// is as fast or faster for every shape (within call overhead at T = 16 with
// few sequences, 1.3x faster at head size 128 with 512 sequences), and 1.35x
// (head size 64) to 1.7x (128) faster from T = 512; below 16 the recurrent
// kernel is as fast or faster (13.8 vs 25.5 us at T = 1, head size 128, 512
// sequences).
constexpr int kChunkedMinTF32 = 16;

wkv7_status_t check_common(int dtype, int B, int H, int K, int V)
{
    if (dtype != WKV7_F32 && dtype != WKV7_BF16) return WKV7_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || K <= 0 || V <= 0) return WKV7_ERR_INVALID_ARG;
    if (K != V || (K != 64 && K != 128)) return WKV7_ERR_UNSUPPORTED;
    if ((long long)B * H > (1ll << 30)) return WKV7_ERR_UNSUPPORTED;
    return WKV7_OK;
}

// gdn: Gated DeltaNet inputs (the chunked kernel takes them with bf16 I/O only).
int choose_path(int dtype, int T, int algo, bool gdn = false)
{
    const bool chunked_ok = dtype == WKV7_BF16 || !gdn;
    if (algo == WKV7_ALGO_RECURRENT) return WKV7_ALGO_RECURRENT;
    if (algo == WKV7_ALGO_CHUNKED) return chunked_ok ? WKV7_ALGO_CHUNKED : -1;
    if (algo != WKV7_ALGO_AUTO) return -1;
    const int min_t = dtype == WKV7_BF16 ? kChunkedMinT : kChunkedMinTF32;
    return chunked_ok && T >= min_t ? WKV7_ALGO_CHUNKED : WKV7_ALGO_RECURRENT;
}

hipError_t launch_path(int path, int dtype, const wkv7::FwdArgs &args, hipStream_t s)
{
    if (path != WKV7_ALGO_CHUNKED) return wkv7::launch_recurrent(dtype, args, s);
    return dtype == WKV7_BF16 ? wkv7::launch_chunked(args, s) : wkv7::launch_chunked_f32(args, s);
}

// Packed sequences: the lengths live on the device, so AUTO cannot look at
// them.  With bf16 the chunked kernel takes any packed batch that has
// tokens: per sequence it is as fast as the recurrent kernel within call
// overhead below 16 tokens and faster from 16 on, so one long sequence among
// many short ones (a mean length under 16) still runs at chunked speed.
int choose_packed_path(int dtype, int total_T, int N, int algo, bool gdn = false)
{
    if (algo == WKV7_ALGO_AUTO && dtype == WKV7_BF16)
        return total_T > 0 ? WKV7_ALGO_CHUNKED : WKV7_ALGO_RECURRENT;
    return choose_path(dtype, total_T / N, algo, gdn);
}

// Launch limits of the backward kernels: the recurrences' grid (2 nbh
// (role, sequence-head) pairs in blocks of eight, each block once per
// 64-column group), and their 32-bit per-lane byte offsets inside one
// 16-token chunk (16 H K elements of at most 4 bytes).
static bool bwd_launch_fits(long long nbh, int H, int K)
{
    return (2 * nbh + 7) / 8 * 8 * (K / 64) <= INT32_MAX && 64ll * H * K <= INT32_MAX;
}

std::atomic<int> g_wait_limit{wkv7::kDefaultWaitLimit};

}  // namespace

int wkv7::current_wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }

// Host-only argument checks of wkv7_bwd apart from the workspace.
int wkv7::check_bwd_args(int dtype, int B, int T, int H, int K, int V, const void *r, const void *w,
                                   const void *k, const void *v, const void *a, const void *b,
                                   const float *initial_state, int n_state, const void *d_o,
                                   const float *d_final_state, const void *dr, const void *dw, const void *dk,
                                   const void *dv, const void *da, const void *db, const float *d_initial_state)
{
    wkv7_status_t st = check_common(dtype, B, H, K, V);
    if (st != WKV7_OK) return st;
    if (T < 0) return WKV7_ERR_INVALID_ARG;
    if ((long long)B * T * H * K > (1ll << 40)) return WKV7_ERR_UNSUPPORTED;
    // launch grids and offsets of the two backward kernels
    if (!bwd_launch_fits((long long)B * H, H, K) || (long long)B * H * ((T + 15) / 16) > INT32_MAX)
        return WKV7_ERR_UNSUPPORTED;
    if (T > 0) {
        const void *req[] = {r, w, k, v, a, b, d_o, dr, dw, dk, dv, da, db};
        for (const void *p : req)
            if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    }
    if (initial_state && n_state != 1 && n_state != B) return WKV7_ERR_INVALID_ARG;
    const void *opt[] = {initial_state, d_final_state, d_initial_state};
    for (const void *p : opt)
        if (p && !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    return WKV7_OK;
}

extern "C" {

int wkv7_set_wait_limit(int polls)
{
    return g_wait_limit.exchange(polls < 0 ? wkv7::kDefaultWaitLimit : polls);
}

int wkv7_version(void) { return 201; }

const char *wkv7_strerror(int status)
{
    switch (status) {
    case WKV7_OK: return "ok";
    case WKV7_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size, dtype or alignment)";
    case WKV7_ERR_UNSUPPORTED: return "unsupported configuration (K == V in {64, 128} required; the chunked Gated DeltaNet path is bf16 only)";
    case WKV7_ERR_HIP: return "HIP kernel launch failed";
    case WKV7_ERR_TOO_LARGE: return "request exceeds the fixed scratch buffer of the allocation-free entry point";
    default: return "unknown status";
    }
}

int wkv7_fwd_path(int dtype, int B, int T, int H, int K, int V, int algo)
{
    if (check_common(dtype, B, H, K, V) != WKV7_OK || T < 0) return -1;
    return choose_path(dtype, T, algo);
}

wkv7_status_t wkv7_fwd(int dtype, int B, int T, int H, int K, int V,
                       const void *r, const void *w, const void *k,
                       const void *v, const void *a, const void *b,
                       const float *initial_state, int n_state, const uint8_t *mask,
                       void *o, float *final_state, int algo, void *stream)
{
    wkv7_status_t st = check_common(dtype, B, H, K, V);
    if (st != WKV7_OK) return st;
    if (T < 0) return WKV7_ERR_INVALID_ARG;
    if ((long long)B * T * H * K > (1ll << 40)) return WKV7_ERR_UNSUPPORTED;
    if (algo != WKV7_ALGO_AUTO && algo != WKV7_ALGO_RECURRENT && algo != WKV7_ALGO_CHUNKED)
        return WKV7_ERR_INVALID_ARG;
    if (T > 0) {
        const void *req[] = {r, w, k, v, a, b, o};
        for (const void *p : req)
            if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    }
    if (initial_state) {
        if (!aligned16(initial_state)) return WKV7_ERR_INVALID_ARG;
        if (n_state != 1 && n_state != B) return WKV7_ERR_INVALID_ARG;
        // a shared state is read by every sequence: writing finals over it races
        if (n_state == 1 && B > 1 && final_state == initial_state) return WKV7_ERR_INVALID_ARG;
    }
    if (final_state && !aligned16(final_state)) return WKV7_ERR_INVALID_ARG;
    const int path = choose_path(dtype, T, algo);
    if (path < 0) return WKV7_ERR_UNSUPPORTED;

    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (!final_state) return WKV7_OK;
        if (!initial_state || n_state == B)
            return wkv7::launch_state_copy(initial_state, final_state, (size_t)B * H * K * V, s) == hipSuccess
                       ? WKV7_OK : WKV7_ERR_HIP;
        const size_t one = (size_t)H * K * V;
        for (int i = 0; i < B; ++i)
            if (wkv7::launch_state_copy(initial_state, final_state + i * one, one, s) != hipSuccess)
                return WKV7_ERR_HIP;
        return WKV7_OK;
    }
    wkv7::FwdArgs args{B, T, H, K, r, w, k, v, a, b, initial_state, mask, o, final_state};
    args.n_state = initial_state ? n_state : 0;
    const hipError_t e = launch_path(path, dtype, args, s);
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

wkv7_status_t wkv7_fwd_varlen(int dtype, int N, int total_T, int H, int K, int V,
                              const int32_t *cu_seqlens,
                              const void *r, const void *w, const void *k,
                              const void *v, const void *a, const void *b,
                              const float *initial_state, int n_state,
                              const int32_t *state_map, const uint8_t *mask,
                              void *o, float *final_state, int algo, void *stream)
{
    wkv7_status_t st = check_common(dtype, N, H, K, V);
    if (st != WKV7_OK) return st;
    if (total_T < 0) return WKV7_ERR_INVALID_ARG;
    if ((long long)total_T * H * K > (1ll << 40)) return WKV7_ERR_UNSUPPORTED;
    if (algo != WKV7_ALGO_AUTO && algo != WKV7_ALGO_RECURRENT && algo != WKV7_ALGO_CHUNKED)
        return WKV7_ERR_INVALID_ARG;
    if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3u)) return WKV7_ERR_INVALID_ARG;
    if (state_map && ((uintptr_t)state_map & 3u)) return WKV7_ERR_INVALID_ARG;
    if (total_T > 0) {
        const void *req[] = {r, w, k, v, a, b, o};
        for (const void *p : req)
            if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    }
    if (initial_state) {
        if (!aligned16(initial_state) || n_state < 1) return WKV7_ERR_INVALID_ARG;
        if (!state_map && n_state != N && n_state != 1) return WKV7_ERR_INVALID_ARG;
        // a pool read through a map, or one shared row, may not be overwritten
        if ((state_map || (n_state == 1 && N > 1)) && final_state == initial_state) return WKV7_ERR_INVALID_ARG;
    }
    if (final_state && !aligned16(final_state)) return WKV7_ERR_INVALID_ARG;
    const int path = choose_packed_path(dtype, total_T, N, algo);
    if (path < 0) return WKV7_ERR_UNSUPPORTED;
    wkv7::FwdArgs args{N, total_T, H, K, r, w, k, v, a, b, initial_state, mask, o, final_state};
    args.cu_seqlens = cu_seqlens;
    args.state_map = state_map;
    args.n_state = initial_state ? n_state : 0;
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = launch_path(path, dtype, args, s);
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

wkv7_status_t wkv7_gdn_fwd(int dtype, int B, int T, int H, int K, int V,
                          const void *q, const void *k, const void *v,
                          const void *g, const void *beta,
                          const float *initial_state, int n_state,
                          void *o, float *final_state, int algo, void *stream)
{
    wkv7_status_t st = check_common(dtype, B, H, K, V);
    if (st != WKV7_OK) return st;
    if (T < 0) return WKV7_ERR_INVALID_ARG;
    if ((long long)B * T * H * K > (1ll << 40)) return WKV7_ERR_UNSUPPORTED;
    if (algo != WKV7_ALGO_AUTO && algo != WKV7_ALGO_RECURRENT && algo != WKV7_ALGO_CHUNKED)
        return WKV7_ERR_INVALID_ARG;
    if (T > 0) {
        const void *req[] = {q, k, v, g, beta, o};
        for (const void *p : req)
            if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    }
    if (initial_state) {
        if (!aligned16(initial_state)) return WKV7_ERR_INVALID_ARG;
        if (n_state != 1 && n_state != B) return WKV7_ERR_INVALID_ARG;
        // a shared state is read by every sequence: writing finals over it races
        if (n_state == 1 && B > 1 && final_state == initial_state) return WKV7_ERR_INVALID_ARG;
    }
    if (final_state && !aligned16(final_state)) return WKV7_ERR_INVALID_ARG;
    const int path = choose_path(dtype, T, algo, true);
    if (path < 0) return WKV7_ERR_UNSUPPORTED;

    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (!final_state) return WKV7_OK;
        const size_t n = (size_t)B * H * K * V;
        if (!initial_state || n_state == B)
            return wkv7::launch_state_copy(initial_state, final_state, n, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
        const size_t one = (size_t)H * K * V;
        for (int i = 0; i < B; ++i)
            if (wkv7::launch_state_copy(initial_state, final_state + i * one, one, s) != hipSuccess)
                return WKV7_ERR_HIP;
        return WKV7_OK;
    }
    // q in the r slot, g in the w slot, beta in the a slot; b and mask unused
    wkv7::FwdArgs args{B, T, H, K, q, g, k, v, beta, nullptr, initial_state, nullptr, o, final_state};
    args.n_state = initial_state ? n_state : 0;
    args.gdn = true;
    const hipError_t e = launch_path(path, dtype, args, s);
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

wkv7_status_t wkv7_gdn_fwd_varlen(int dtype, int N, int total_T, int H, int K, int V,
                                  const int32_t *cu_seqlens,
                                  const void *q, const void *k, const void *v,
                                  const void *g, const void *beta,
                                  const float *initial_state, int n_state,
                                  const int32_t *state_map,
                                  void *o, float *final_state, int algo, void *stream)
{
    wkv7_status_t st = check_common(dtype, N, H, K, V);
    if (st != WKV7_OK) return st;
    if (total_T < 0) return WKV7_ERR_INVALID_ARG;
    if ((long long)total_T * H * K > (1ll << 40)) return WKV7_ERR_UNSUPPORTED;
    if (algo != WKV7_ALGO_AUTO && algo != WKV7_ALGO_RECURRENT && algo != WKV7_ALGO_CHUNKED)
        return WKV7_ERR_INVALID_ARG;
    if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3u)) return WKV7_ERR_INVALID_ARG;
    if (state_map && ((uintptr_t)state_map & 3u)) return WKV7_ERR_INVALID_ARG;
    if (total_T > 0) {
        const void *req[] = {q, k, v, g, beta, o};
        for (const void *p : req)
            if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    }
    if (initial_state) {
        if (!aligned16(initial_state) || n_state < 1) return WKV7_ERR_INVALID_ARG;
        if (!state_map && n_state != N && n_state != 1) return WKV7_ERR_INVALID_ARG;
        // a pool read through a map, or one shared row, may not be overwritten
        if ((state_map || (n_state == 1 && N > 1)) && final_state == initial_state) return WKV7_ERR_INVALID_ARG;
    }
    if (final_state && !aligned16(final_state)) return WKV7_ERR_INVALID_ARG;
    const int path = choose_packed_path(dtype, total_T, N, algo, true);
    if (path < 0) return WKV7_ERR_UNSUPPORTED;
    wkv7::FwdArgs args{N, total_T, H, K, q, g, k, v, beta, nullptr, initial_state, nullptr, o, final_state};
    args.cu_seqlens = cu_seqlens;
    args.state_map = state_map;
    args.n_state = initial_state ? n_state : 0;
    args.gdn = true;
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = launch_path(path, dtype, args, s);
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

size_t wkv7_bwd_workspace_bytes(int B, int T, int H, int K, int V)
{
    if (check_common(WKV7_F32, B, H, K, V) != WKV7_OK || T < 0) return 0;
    return wkv7::bwd_workspace_bytes(B, T, H, K);
}

wkv7_status_t wkv7_bwd(int dtype, int B, int T, int H, int K, int V,
                       const void *r, const void *w, const void *k,
                       const void *v, const void *a, const void *b,
                       const float *initial_state, int n_state, const uint8_t *mask,
                       const void *d_o, const float *d_final_state,
                       void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                       float *d_initial_state, void *workspace, size_t workspace_bytes,
                       void *stream)
{
    const wkv7_status_t st = (wkv7_status_t)wkv7::check_bwd_args(
        dtype, B, T, H, K, V, r, w, k, v, a, b, initial_state, n_state, d_o, d_final_state, dr, dw, dk, dv, da, db,
        d_initial_state);
    if (st != WKV7_OK) return st;
    if (T > 0) {
        if (!workspace || !aligned16(workspace)) return WKV7_ERR_INVALID_ARG;
        if (workspace_bytes < wkv7::bwd_workspace_bytes(B, T, H, K)) return WKV7_ERR_INVALID_ARG;
    }
    const bool shared = initial_state && n_state == 1 && B > 1;

    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (!d_initial_state) return WKV7_OK;
        const size_t per = (size_t)H * K * V;
        hipError_t e = shared ? wkv7::launch_state_sum(d_final_state, d_initial_state, B, per, s)
                              : wkv7::launch_state_copy(d_final_state, d_initial_state, (size_t)B * per, s);
        return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
    }
    // A shared initial state's gradient is the sum over the B sequences:
    // per-sequence gradients go to the workspace's tail, then one ordered sum.
    float *ds0_rows = shared ? (float *)((char *)workspace + (wkv7::bwd_checkpoint_bytes(B, T, H, K) + 255) / 256 * 256)
                             : d_initial_state;
    wkv7::BwdArgs args{B, T, H, K, r, w, k, v, a, b, initial_state, mask, d_o, d_final_state,
                       dr, dw, dk, dv, da, db, d_initial_state ? ds0_rows : nullptr, workspace};
    args.n_state = initial_state ? n_state : 0;
    hipError_t e = wkv7::launch_backward(dtype, args, s);
    if (e == hipSuccess && shared && d_initial_state)
        e = wkv7::launch_state_sum(ds0_rows, d_initial_state, B, (size_t)H * K * V, s);
    return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

size_t wkv7_bwd_varlen_workspace_bytes(int N, int total_T, int H, int K, int V)
{
    if (check_common(WKV7_F32, N, H, K, V) != WKV7_OK || total_T < 0) return 0;
    return wkv7::bwd_varlen_workspace_bytes(N, total_T, H, K);
}

wkv7_status_t wkv7_bwd_varlen(int dtype, int N, int total_T, int H, int K, int V,
                              const int32_t *cu_seqlens,
                              const void *r, const void *w, const void *k,
                              const void *v, const void *a, const void *b,
                              const float *initial_state, int n_state, const int32_t *state_map,
                              const uint8_t *mask, const void *d_o, const float *d_final_state,
                              void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                              float *d_initial_state, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    wkv7_status_t st = check_common(dtype, N, H, K, V);
    if (st != WKV7_OK) return st;
    if (total_T < 0) return WKV7_ERR_INVALID_ARG;
    if ((long long)total_T * H * K > (1ll << 40)) return WKV7_ERR_UNSUPPORTED;
    // launch grids and offsets of the two backward kernels (H per chunk of the capacity)
    if (!bwd_launch_fits((long long)N * H, H, K) || wkv7::bwd_varlen_chunk_capacity(N, total_T) * H > INT32_MAX)
        return WKV7_ERR_UNSUPPORTED;
    if (total_T > 0) {
        const void *req[] = {r, w, k, v, a, b, d_o, dr, dw, dk, dv, da, db, workspace};
        for (const void *p : req)
            if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
        if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3)) return WKV7_ERR_INVALID_ARG;
        if (workspace_bytes < wkv7::bwd_varlen_workspace_bytes(N, total_T, H, K)) return WKV7_ERR_INVALID_ARG;
    }
    if (initial_state) {
        if (n_state < 1) return WKV7_ERR_INVALID_ARG;
        if (!state_map && n_state != N && n_state != 1) return WKV7_ERR_INVALID_ARG;
    }
    if (state_map && ((uintptr_t)state_map & 3)) return WKV7_ERR_INVALID_ARG;
    const void *opt[] = {initial_state, d_final_state, d_initial_state};
    for (const void *p : opt)
        if (p && !aligned16(p)) return WKV7_ERR_INVALID_ARG;

    hipStream_t s = (hipStream_t)stream;
    if (total_T == 0) {
        // every sequence is empty: its initial-state gradient is its final-state gradient
        if (!d_initial_state) return WKV7_OK;
        const size_t n = (size_t)N * H * K * V;
        return wkv7::launch_state_copy(d_final_state, d_initial_state, n, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
    }
    wkv7::BwdArgs args{N, total_T, H, K, r, w, k, v, a, b, initial_state, mask, d_o, d_final_state,
                       dr, dw, dk, dv, da, db, d_initial_state, workspace};
    args.cu_seqlens = cu_seqlens;
    args.state_map = state_map;
    args.n_state = initial_state ? n_state : 0;
    return wkv7::launch_backward(dtype, args, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

size_t wkv7_gdn_bwd_workspace_bytes(int B, int T, int H, int K, int V)
{
    if (check_common(WKV7_F32, B, H, K, V) != WKV7_OK || T < 0) return 0;
    return wkv7::gdn_bwd_workspace_bytes(B, T, H, K);
}

wkv7_status_t wkv7_gdn_bwd(int dtype, int B, int T, int H, int K, int V,
                           const void *q, const void *k, const void *v,
                           const void *g, const void *beta,
                           const float *initial_state, int n_state,
                           const void *d_o, const float *d_final_state,
                           void *dq, void *dk, void *dv, void *dg, void *dbeta,
                           float *d_initial_state, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    wkv7_status_t st = check_common(dtype, B, H, K, V);
    if (st != WKV7_OK) return st;
    if (T < 0) return WKV7_ERR_INVALID_ARG;
    if ((long long)B * T * H * K > (1ll << 40)) return WKV7_ERR_UNSUPPORTED;
    // launch grids and offsets of the WKV7 backward it runs
    if (!bwd_launch_fits((long long)B * H, H, K) || (long long)B * H * ((T + 15) / 16) > INT32_MAX)
        return WKV7_ERR_UNSUPPORTED;
    if (T > 0) {
        const void *req[] = {q, k, v, g, beta, d_o, dq, dk, dv, dg, dbeta, workspace};
        for (const void *p : req)
            if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
        if (workspace_bytes < wkv7::gdn_bwd_workspace_bytes(B, T, H, K)) return WKV7_ERR_INVALID_ARG;
    }
    if (initial_state && n_state != 1 && n_state != B) return WKV7_ERR_INVALID_ARG;
    const void *opt[] = {initial_state, d_final_state, d_initial_state};
    for (const void *p : opt)
        if (p && !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    const int rows = initial_state ? n_state : B;   // rows of d_initial_state

    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (!d_initial_state) return WKV7_OK;
        const size_t per = (size_t)H * K * V;
        hipError_t e = rows == B ? wkv7::launch_state_copy(d_final_state, d_initial_state, (size_t)B * per, s)
                                 : wkv7::launch_state_sum(d_final_state, d_initial_state, B, per, s);
        return e == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
    }
    wkv7::GdnBwdArgs args{B, T, H, K, q, k, v, g, beta, initial_state, rows, d_o, d_final_state,
                          dq, dk, dv, dg, dbeta, d_initial_state, workspace};
    return wkv7::launch_gdn_backward(dtype, args, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

size_t wkv7_gdn_bwd_varlen_workspace_bytes(int N, int total_T, int H, int K, int V)
{
    return wkv7_bwd_varlen_workspace_bytes(N, total_T, H, K, V);
}

wkv7_status_t wkv7_gdn_bwd_varlen(int dtype, int N, int total_T, int H, int K, int V,
                                  const int32_t *cu_seqlens,
                                  const void *q, const void *k, const void *v,
                                  const void *g, const void *beta,
                                  const float *initial_state, int n_state, const int32_t *state_map,
                                  const void *d_o, const float *d_final_state,
                                  void *dq, void *dk, void *dv, void *dg, void *dbeta,
                                  float *d_initial_state, void *workspace, size_t workspace_bytes,
                                  void *stream)
{
    wkv7_status_t st = check_common(dtype, N, H, K, V);
    if (st != WKV7_OK) return st;
    if (total_T < 0) return WKV7_ERR_INVALID_ARG;
    if ((long long)total_T * H * K > (1ll << 40)) return WKV7_ERR_UNSUPPORTED;
    if (!bwd_launch_fits((long long)N * H, H, K) || wkv7::bwd_varlen_chunk_capacity(N, total_T) * H > INT32_MAX)
        return WKV7_ERR_UNSUPPORTED;
    if (total_T > 0) {
        const void *req[] = {q, k, v, g, beta, d_o, dq, dk, dv, dg, dbeta, workspace};
        for (const void *p : req)
            if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
        if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3)) return WKV7_ERR_INVALID_ARG;
        if (workspace_bytes < wkv7::bwd_varlen_workspace_bytes(N, total_T, H, K)) return WKV7_ERR_INVALID_ARG;
    }
    if (initial_state) {
        if (n_state < 1) return WKV7_ERR_INVALID_ARG;
        if (!state_map && n_state != N && n_state != 1) return WKV7_ERR_INVALID_ARG;
    }
    if (state_map && ((uintptr_t)state_map & 3)) return WKV7_ERR_INVALID_ARG;
    const void *opt[] = {initial_state, d_final_state, d_initial_state};
    for (const void *p : opt)
        if (p && !aligned16(p)) return WKV7_ERR_INVALID_ARG;

    hipStream_t s = (hipStream_t)stream;
    if (total_T == 0) {
        if (!d_initial_state) return WKV7_OK;
        const size_t n = (size_t)N * H * K * V;
        return wkv7::launch_state_copy(d_final_state, d_initial_state, n, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
    }
    // q in the r slot, g in the w slot, beta in the a slot (the kernels' Gated DeltaNet mode)
    wkv7::BwdArgs args{N, total_T, H, K, q, g, k, v, beta, nullptr, initial_state, nullptr, d_o, d_final_state,
                       dq, dg, dk, dv, dbeta, nullptr, d_initial_state, workspace};
    args.gdn = true;
    args.cu_seqlens = cu_seqlens;
    args.state_map = state_map;
    args.n_state = initial_state ? n_state : 0;
    return wkv7::launch_backward(dtype, args, s) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

wkv7_status_t wkv7_step(int dtype, int B, int H, int K, int V,
                        const void *r, const void *w, const void *k,
                        const void *v, const void *a, const void *b,
                        float *state, void *o, void *stream)
{
    wkv7_status_t st = check_common(dtype, B, H, K, V);
    if (st != WKV7_OK) return st;
    if (4ll * B * H > INT32_MAX) return WKV7_ERR_UNSUPPORTED;   // up to four waves per (b, h)
    const void *req[] = {r, w, k, v, a, b, state, o};
    for (const void *p : req)
        if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    wkv7::StepArgs args{B, H, K, r, w, k, v, a, b, state, o};
    return wkv7::launch_step(dtype, args, (hipStream_t)stream) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

wkv7_status_t wkv7_gdn_step(int dtype, int B, int H, int K, int V,
                            const void *q, const void *k, const void *v,
                            const void *g, const void *beta,
                            const float *state_in, int n_state, float *state_out,
                            void *o, void *stream)
{
    wkv7_status_t st = check_common(dtype, B, H, K, V);
    if (st != WKV7_OK) return st;
    if (4ll * B * H > INT32_MAX) return WKV7_ERR_UNSUPPORTED;   // up to four waves per (b, h)
    const void *req[] = {q, k, v, g, beta, state_out, o};
    for (const void *p : req)
        if (!p || !aligned16(p)) return WKV7_ERR_INVALID_ARG;
    if (state_in) {
        if (!aligned16(state_in)) return WKV7_ERR_INVALID_ARG;
        if (n_state != 1 && n_state != B) return WKV7_ERR_INVALID_ARG;
        // a shared state read by every sequence may not be overwritten by them
        if (n_state == 1 && B > 1 && state_in == state_out) return WKV7_ERR_INVALID_ARG;
    }
    wkv7::StepArgs args{B, H, K, q, g, k, v, beta, nullptr, state_out, o};
    args.gdn = true;
    args.state_in = state_in;
    args.n_state_in = state_in ? n_state : 0;
    return wkv7::launch_step(dtype, args, (hipStream_t)stream) == hipSuccess ? WKV7_OK : WKV7_ERR_HIP;
}

}  // extern "C"

namespace wkv7 {

__global__ void state_copy_kernel(const float *__restrict__ src, float *__restrict__ dst, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_state_copy(const float *s0, float *sf, size_t n, hipStream_t stream)
{
    if (s0 == sf) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, s0, sf, n);
    return hipGetLastError();
}

}  // namespace wkv7

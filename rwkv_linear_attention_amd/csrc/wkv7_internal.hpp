// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

// Polls a wave of the chunked forward makes on a hand-off counter before it
// gives up and poisons its results with NaN: the default, and the value in
// force for new launches (set by wkv7_set_wait_limit).
constexpr int kDefaultWaitLimit = 1 << 20;
int current_wait_limit();

// Fixed-length form: B sequences of T tokens, [B,T,H,D] arrays,
// cu_seqlens == state_map == nullptr, n_state == B.  Packed form: B
// sequences with token ranges [cu_seqlens[n], cu_seqlens[n+1]) of a
// [T,H,D] token axis (T = total tokens), initial state row state_map[n]
// of an [n_state,H,D,D] pool (state_map == nullptr: row n).
struct FwdArgs {
    int B, T, H, D;                      // D = K = V
    const void *r, *w, *k, *v, *a, *b;   // I/O dtype
    const float *s0;                     // state pool [n_state,H,D,D] or nullptr
    const uint8_t *mask;                 // one byte per token or nullptr
    void *o;                             // I/O dtype
    float *sf;                           // [B,H,D,D] or nullptr
    const int32_t *cu_seqlens = nullptr; // device, [B+1]
    const int32_t *state_map = nullptr;  // device, [B]
    int n_state = 0;                     // 1 with no state_map: one shared state
    // Gated DeltaNet inputs in the same slots: r = q, k = k, v = v,
    // w = gate g and a = strength beta, both one value per token and head.
    bool gdn = false;
};

// Backward (fixed-length form): gradients of the forward for upstream d_o
// [B,T,H,D] and d_sf [B,H,D,D] (or nullptr); dr..db in the I/O dtype, d_s0
// fp32 [B,H,D,D] per sequence (or nullptr), also when n_state == 1 (one
// initial state shared by every sequence).  ws: workspace of
// bwd_workspace_bytes(B,T,H,D) bytes.
struct BwdArgs {
    int B, T, H, D;
    const void *r, *w, *k, *v, *a, *b;
    const float *s0;
    const uint8_t *mask;
    const void *d_o;
    const float *d_sf;
    void *dr, *dw, *dk, *dv, *da, *db;
    float *d_s0;
    void *ws;
    // Gated DeltaNet: r = q, w = g and a = beta ([B,T,H]), b and mask unused;
    // dr = dq, dw = dg and da = dbeta ([B,T,H]), db unused.
    bool gdn = false;
    // Packed form: B sequences with token ranges [cu_seqlens[n],
    // cu_seqlens[n+1]) of a [T,H,D] token axis (T = total tokens), initial
    // state row state_map[n] of an [n_state,H,D,D] pool (state_map ==
    // nullptr: row n); d_sf and d_s0 are [B,H,D,D] (per sequence).  ws:
    // bwd_varlen_workspace_bytes(B,T,H,D) bytes.
    const int32_t *cu_seqlens = nullptr;
    const int32_t *state_map = nullptr;
    int n_state = 0;
};
// Fixed-length form: the checkpoints (two fp32 states per 16-token chunk
// and sequence), then B per-sequence initial-state gradients at a 256-byte
// aligned offset (used to sum the gradient of a shared initial state).
size_t bwd_checkpoint_bytes(int B, int T, int H, int D);
size_t bwd_workspace_bytes(int B, int T, int H, int D);
// Packed form: chunk capacity ceil(T/16) + B (an upper bound on the sum of
// the sequences' chunk counts), two fp32 states per chunk and head, then the
// per-sequence chunk offsets.
long long bwd_varlen_chunk_capacity(int B, int T);
size_t bwd_varlen_workspace_bytes(int B, int T, int H, int D);

// Gated DeltaNet backward (fixed-length form): q, k [B,T,H,D], v and d_o
// [B,T,H,D], g and beta [B,T,H], all in the I/O dtype; s0 [n_state,H,D,D]
// (n_state 1 or B) or nullptr; d_sf [B,H,D,D] or nullptr; dq .. dbeta in the
// I/O dtype; d_s0 [n_state,H,D,D] (B rows without s0) or nullptr.
// ws: workspace of gdn_bwd_workspace_bytes(B,T,H,D) bytes.
struct GdnBwdArgs {
    int B, T, H, D;
    const void *q, *k, *v, *g, *beta;
    const float *s0;
    int n_state;
    const void *d_o;
    const float *d_sf;
    void *dq, *dk, *dv, *dg, *dbeta;
    float *d_s0;
    void *ws;
};
size_t gdn_bwd_workspace_bytes(int B, int T, int H, int D);

struct StepArgs {
    int B, H, D;
    const void *r, *w, *k, *v, *a, *b;   // [B,H,D]
    float *state;                        // [B,H,D,D], in place (Gated DeltaNet: written)
    void *o;                             // [B,H,D]
    // Gated DeltaNet decode: r = q, w = g and a = beta ([B,H]); the state is
    // read from state_in ([n_state_in,H,D,D], n_state_in 1 or B, or nullptr
    // for zeros) and written to state.
    bool gdn = false;
    const float *state_in = nullptr;
    int n_state_in = 0;
};

// Host-only argument checks of wkv7_bwd apart from the workspace (status
// values of wkv7_status_t).
int check_bwd_args(int dtype, int B, int T, int H, int K, int V, const void *r, const void *w, const void *k,
                   const void *v, const void *a, const void *b, const float *initial_state, int n_state,
                   const void *d_o, const float *d_final_state, const void *dr, const void *dw, const void *dk,
                   const void *dv, const void *da, const void *db, const float *d_initial_state);

// dtype: 0 = fp32, 1 = bf16 (values of wkv7_dtype_t).
hipError_t launch_recurrent(int dtype, const FwdArgs &args, hipStream_t stream);
hipError_t launch_chunked(const FwdArgs &args, hipStream_t stream);     // bf16 I/O
hipError_t launch_chunked_f32(const FwdArgs &args, hipStream_t stream); // fp32 I/O, not Gated DeltaNet
hipError_t launch_step(int dtype, const StepArgs &args, hipStream_t stream);
hipError_t launch_backward(int dtype, const BwdArgs &args, hipStream_t stream);
hipError_t launch_gdn_backward(int dtype, const GdnBwdArgs &args, hipStream_t stream);
// dst = sum of the B states of src ([B][per] floats; src == nullptr: zeros).
hipError_t launch_state_sum(const float *src, float *dst, int B, size_t per, hipStream_t stream);
// final_state = initial_state (or zeros) for T == 0.
hipError_t launch_state_copy(const float *s0, float *sf, size_t n, hipStream_t stream);

}  // namespace wkv7

/*
 * wkv7.h -- C ABI of libwkv7.so: the RWKV-7 WKV7 generalized-delta-rule
 * forward and single-token decode on MI355X (gfx950).
 *
 * Operation (rwkv-ops README, PyPI rwkv-ops 0.7.4 and rwkv_ops 0.9.0 METADATA,
 * section "rwkv7op 使用方法", docstring of generalized_delta_rule; the
 * single-token form is section "rwkv7_op_rnn 使用方法"):
 *
 *   per sequence b and head h, with a K x V fp32 state S (rows K, columns V):
 *     if mask[b,t] != 0:  S = diag(exp(w_t)) S + a_t (b_t^T S) + k_t v_t^T
 *     o_t = S^T r_t
 *   w is the decay in log space (normally <= 0).  A token whose mask byte is
 *   0 leaves S unchanged and still emits o_t = S^T r_t.  The update formula
 *   itself is not printed on those pages; this is the generalized delta rule
 *   reading (low-rank term from the state before this token's decay, a on the
 *   K side, b contracting with the state, output from the updated state, no
 *   scale on r, no bonus term).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous,
 *     16-byte aligned.  The caller owns every buffer; the library allocates
 *     no device memory and keeps no pointer after the call returns.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream).  No call synchronises; results are ready when the
 *     stream reaches them.
 *   - Every call returns a wkv7_status_t.  Nothing aborts or throws.  Size,
 *     pointer, dtype and alignment checks run on the host before any HIP
 *     call, so they work on a machine without a GPU.  Data values are not
 *     inspected: NaN / Inf propagate.
 *   - Supported sizes: K == V, K in {64, 128}.
 *   - Thread safety: the library holds no mutable global state apart from
 *     the wait-limit test hook (wkv7_set_wait_limit); concurrent calls on
 *     different streams are independent.
 */
#ifndef WKV7_H
#define WKV7_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WKV7_F32 = 0,   /* fp32 inputs and output (the state is fp32 always)   */
    WKV7_BF16 = 1   /* bf16 inputs and output; fp32 state                   */
} wkv7_dtype_t;

typedef enum {
    WKV7_ALGO_AUTO = 0,       /* library chooses (see wkv7_fwd)            */
    WKV7_ALGO_RECURRENT = 1,  /* token-by-token fp32 recurrence            */
    WKV7_ALGO_CHUNKED = 2     /* 16-token chunks on the matrix cores        */
} wkv7_algo_t;

typedef enum {
    WKV7_OK = 0,
    WKV7_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size, misaligned */
    WKV7_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
    WKV7_ERR_HIP = 3,         /* a HIP launch failed                         */
    WKV7_ERR_TOO_LARGE = 4    /* exceeds the fixed scratch of wkv7_bwd_noalloc */
} wkv7_status_t;

/*
 * wkv7_fwd -- forward over whole sequences (section "rwkv7op 使用方法").
 *
 *   dtype          WKV7_F32 or WKV7_BF16: element type of r,w,k,v,a,b and o.
 *   B, T, H        batch, sequence length, heads.  B, H >= 1; T >= 0.
 *   K, V           key and value head size; K == V in {64, 128}.
 *   r,w,k,a,b      [B,T,H,K] dtype (seq-first layout).  Read only.
 *   v              [B,T,H,V] dtype.  Read only.
 *   initial_state  [n_state,H,K,V] fp32, or NULL for a zero state.  Read
 *                  only.  n_state = 1 is one state shared by all B
 *                  sequences (the (1,H,K,V) initial state of the rwkv-ops
 *                  README argument tables, sections "gdn_recurrent 使用方法"
 *                  and "rwkv7op_sane 使用方法").
 *   n_state        B or 1 when initial_state is given; ignored otherwise.
 *   mask           [B,T] uint8 (nonzero = update, 0 = keep), or NULL for
 *                  all tokens updating.  Read only.
 *   o              [B,T,H,V] dtype.  Written (every element).
 *   final_state    [B,H,K,V] fp32, or NULL to skip it.  Written.  It may be
 *                  the same buffer as initial_state (in-place state passing)
 *                  when n_state == B (or B == 1); any other overlap between
 *                  buffers is undefined.
 *   algo           WKV7_ALGO_AUTO picks the chunked kernel when the
 *                  sequences are long enough to amortise it (T >= 16; bf16
 *                  I/O runs on bf16 matrix cores with fp32 accumulation,
 *                  fp32 I/O on fp32 matrix cores) and the recurrent kernel
 *                  otherwise.
 *   stream         hipStream_t to enqueue on.
 * With T == 0, o is empty and final_state (if given) receives initial_state
 * in every row (zeros when initial_state is NULL).
 */
wkv7_status_t wkv7_fwd(int dtype, int B, int T, int H, int K, int V,
                       const void *r, const void *w, const void *k,
                       const void *v, const void *a, const void *b,
                       const float *initial_state, int n_state, const uint8_t *mask,
                       void *o, float *final_state, int algo, void *stream);

/*
 * wkv7_fwd_varlen -- forward over N variable-length sequences packed back to
 * back along one token axis, each starting from an entry of a pool of
 * initial states.  Packed variable-length input follows the rwkv-fla page
 * (its news note on kernels with variable-length inputs); the state index
 * per sample follows the state_map argument of the rwkv-ops README
 * operator interface (an index per sample into an [n_state, H, K, V]
 * initial state; n_state = 1 shares one state).  Sequence n computes
 * exactly what wkv7_fwd computes for one sequence of length
 * cu_seqlens[n+1] - cu_seqlens[n].
 *
 *   dtype          as for wkv7_fwd.
 *   N              number of sequences, >= 1.
 *   total_T        length of the packed token axis, >= 0.
 *   H, K, V        as for wkv7_fwd.
 *   cu_seqlens     DEVICE int32 [N+1], 4-byte aligned: sequence n owns tokens
 *                  [cu_seqlens[n], cu_seqlens[n+1]).  Expected nondecreasing
 *                  from 0 to total_T; the kernels clamp every offset into
 *                  [0, total_T] and treat a decreasing pair as an empty
 *                  sequence, so malformed offsets give wrong results but
 *                  never an out-of-bounds access.  Read only.
 *   r,w,k,a,b      [total_T,H,K] dtype.  Read only.
 *   v              [total_T,H,V] dtype.  Read only.
 *   initial_state  [n_state,H,K,V] fp32 pool, or NULL for zero states.
 *   n_state        rows of the pool (>= 1 when initial_state is given).
 *   state_map      DEVICE int32 [N], 4-byte aligned, or NULL.  Sequence n
 *                  starts from pool row state_map[n]; an entry outside
 *                  [0, n_state) means a zero state.  NULL means row n, which
 *                  requires n_state == N, or n_state == 1 (one row shared
 *                  by every sequence), when initial_state is given.
 *   mask           [total_T] uint8 (nonzero = update), or NULL.
 *   o              [total_T,H,V] dtype.  Written at every token of every
 *                  sequence (tokens outside all sequences are not written).
 *   final_state    [N,H,K,V] fp32, or NULL.  Written.  May alias
 *                  initial_state only when state_map is NULL and the pool
 *                  has a row per sequence.
 *   algo           as for wkv7_fwd; under AUTO with bf16 the chunked kernel
 *                  takes every packed batch with total_T > 0 (the lengths
 *                  are on the device, so the choice cannot depend on them,
 *                  and a batch of short sequences costs the chunked kernel
 *                  no more than the recurrent one beyond call overhead).
 *   stream         hipStream_t to enqueue on.
 */
wkv7_status_t wkv7_fwd_varlen(int dtype, int N, int total_T, int H, int K, int V,
                              const int32_t *cu_seqlens,
                              const void *r, const void *w, const void *k,
                              const void *v, const void *a, const void *b,
                              const float *initial_state, int n_state,
                              const int32_t *state_map, const uint8_t *mask,
                              void *o, float *final_state, int algo, void *stream);

/*
 * wkv7_gdn_fwd -- Gated DeltaNet forward over whole sequences (rwkv-ops
 * README, section "gdn_recurrent 使用方法", argument table of
 * gated_delta_net_recurrent; the chunked form "gdn_chunk 使用方法" computes
 * the same).  Per sequence and head, with a K x V fp32 state S:
 *     qn = q_t / sqrt(|q_t|^2 + 1e-6),  kn = k_t / sqrt(|k_t|^2 + 1e-6)
 *     S  = e^{g_t} S,  then  S = S + beta_t kn (v_t - S^T kn)^T
 *        (that is, S = e^{g_t} (I - beta_t kn kn^T) S + beta_t kn v_t^T)
 *     o_t = S^T qn
 * The pages name the inputs, the internal L2 normalisation of q and k, the
 * log-space gate g and the strength beta in (0, 1); the update itself is not
 * printed there and is read as the gated delta rule (decay first, then the
 * delta-rule correction and write, no scale on q; 1e-6 inside the norm is
 * this library's choice).  It is the generalized delta rule of wkv7_fwd with
 * r = qn, w = g on every channel, k = beta kn, a = -e^g beta kn, b = kn.
 *
 *   dtype          WKV7_F32 or WKV7_BF16: element type of q,k,v,g,beta and o.
 *   B, T, H, K, V  as for wkv7_fwd; K == V in {64, 128}.
 *   q, k           [B,T,H,K] dtype, raw (normalised inside).  Read only.
 *   v              [B,T,H,V] dtype.  Read only.
 *   g              [B,T,H] dtype, log-space gate (normally <= 0).  Read only.
 *   beta           [B,T,H] dtype, write strength.  Read only.
 *   initial_state  [n_state,H,K,V] fp32 with n_state 1 (shared by all B
 *                  sequences) or B, or NULL for a zero state.  Read only.
 *   n_state        1 or B when initial_state is given; ignored otherwise.
 *   o              [B,T,H,V] dtype.  Written.
 *   final_state    [B,H,K,V] fp32, or NULL.  Written.  May be the same buffer
 *                  as initial_state only when n_state == B (or B == 1).
 *   algo           as for wkv7_fwd, except that the chunked kernel takes
 *                  bf16 only: AUTO runs fp32 on the recurrent kernel, and
 *                  WKV7_ALGO_CHUNKED with fp32 returns WKV7_ERR_UNSUPPORTED.
 *   stream         hipStream_t to enqueue on.
 */
wkv7_status_t wkv7_gdn_fwd(int dtype, int B, int T, int H, int K, int V,
                           const void *q, const void *k, const void *v,
                           const void *g, const void *beta,
                           const float *initial_state, int n_state,
                           void *o, float *final_state, int algo, void *stream);

/*
 * wkv7_gdn_fwd_varlen -- Gated DeltaNet forward over N variable-length
 * sequences packed on one token axis, each starting from an entry of a pool
 * of initial states: wkv7_gdn_fwd's operation with wkv7_fwd_varlen's packing
 * and state indexing (same argument meanings; g and beta are [total_T,H]).
 * With state_map NULL the pool has N rows (row n) or one shared row.  A
 * mapped or shared pool may not be the final_state buffer.
 */
wkv7_status_t wkv7_gdn_fwd_varlen(int dtype, int N, int total_T, int H, int K, int V,
                                  const int32_t *cu_seqlens,
                                  const void *q, const void *k, const void *v,
                                  const void *g, const void *beta,
                                  const float *initial_state, int n_state,
                                  const int32_t *state_map,
                                  void *o, float *final_state, int algo, void *stream);

/*
 * wkv7_bwd -- gradients of wkv7_fwd (rwkv-ops README, section
 * "rwkv7op 使用方法": generalized_delta_rule is the trainable entry; the
 * derivative follows from the recurrence by the chain rule).  For upstream
 * gradients d_o (of every output) and d_final_state (of the final state) it
 * returns the gradients of r, w, k, v, a, b and of the initial state.  A
 * token whose mask byte is 0 receives zero gradient for w, k, v, a and b
 * (its r still receives S_{t-1} d_o_t).  The forward is recomputed inside
 * (fp32 state checkpoints every 16 tokens), so only the forward's inputs are
 * needed; all arithmetic is fp32, also for bf16 I/O.
 *
 *   dtype          WKV7_F32 or WKV7_BF16: element type of r,w,k,v,a,b, d_o
 *                  and of the gradients dr..db.
 *   B,T,H,K,V      as for wkv7_fwd; K == V in {64, 128}.
 *   r,w,k,v,a,b    the forward's inputs, as for wkv7_fwd.  Read only.
 *   initial_state  [n_state,H,K,V] fp32 or NULL (zeros).  Read only.
 *   n_state        B or 1 (one state shared by all B sequences) when
 *                  initial_state is given; ignored otherwise.
 *   mask           [B,T] uint8 or NULL.  Read only.
 *   d_o            [B,T,H,V] dtype.  Read only.
 *   d_final_state  [B,H,K,V] fp32 or NULL (zero).  Read only.
 *   dr,dw,dk,da,db [B,T,H,K] dtype; dv [B,T,H,V] dtype.  Written (every element).
 *   d_initial_state [n_state,H,K,V] fp32 ([B,H,K,V] without initial_state:
 *                  the gradient of the zero start) or NULL (not written).
 *                  Written.  With a shared state it is the sum over the B
 *                  sequences, taken in sequence order (deterministic).
 *   workspace      DEVICE buffer of at least wkv7_bwd_workspace_bytes(B,T,H,K,V)
 *                  bytes, 16-byte aligned, owned by the caller; contents on
 *                  entry are ignored and on return are unspecified.  May be
 *                  NULL when T == 0.
 *   stream         hipStream_t to enqueue on.
 * Output buffers must not overlap any input or each other.  With T == 0,
 * d_initial_state receives d_final_state (summed over B for a shared state;
 * zeros when NULL).  Returns WKV7_ERR_UNSUPPORTED when H*K reaches 2^25 (the
 * kernels address one 16-token chunk with 32-bit offsets) or a launch grid
 * would exceed 2^31 - 1 workgroups; the same limits hold for every backward
 * entry point.
 */
wkv7_status_t wkv7_bwd(int dtype, int B, int T, int H, int K, int V,
                       const void *r, const void *w, const void *k,
                       const void *v, const void *a, const void *b,
                       const float *initial_state, int n_state, const uint8_t *mask,
                       const void *d_o, const float *d_final_state,
                       void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                       float *d_initial_state, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Workspace bytes wkv7_bwd needs: 4 B 2 ceil(T/16) H K V (two fp32 states
 * per 16-token chunk and sequence) rounded up to a multiple of 256, plus
 * 4 B H K V (per-sequence gradients of a shared initial state), or 0 for
 * arguments wkv7_bwd would reject. */
size_t wkv7_bwd_workspace_bytes(int B, int T, int H, int K, int V);

/*
 * wkv7_bwd_varlen -- gradients of wkv7_fwd_varlen (N packed sequences; the
 * pages' trainable generalized_delta_rule takes an initial state with N
 * rows, one per sequence, and only its head-first layout excludes variable
 * lengths: rwkv-ops README, section "rwkv7op 使用方法").  Sequence n gets
 * exactly the gradients wkv7_bwd gives for that one sequence.
 *
 *   dtype, N, total_T, H, K, V, cu_seqlens, r,w,k,v,a,b, initial_state,
 *   n_state, state_map, mask
 *                  as for wkv7_fwd_varlen.  Read only.
 *   d_o            [total_T,H,V] dtype.  Read only.
 *   d_final_state  [N,H,K,V] fp32 or NULL (zero).  Read only.
 *   dr,dw,dk,da,db [total_T,H,K] dtype; dv [total_T,H,V] dtype.  Written at
 *                  every token of every sequence; tokens outside all
 *                  sequences are not written.
 *   d_initial_state [N,H,K,V] fp32 or NULL: row n is the gradient of the
 *                  state sequence n started from (the gradient of a pool row
 *                  is the sum of the rows of the sequences mapped to it,
 *                  which is left to the caller).  Written.
 *   workspace      DEVICE buffer of at least
 *                  wkv7_bwd_varlen_workspace_bytes(N,total_T,H,K,V) bytes,
 *                  16-byte aligned, owned by the caller; contents on entry
 *                  are ignored, on return unspecified.  May be NULL when
 *                  total_T == 0.
 *   stream         hipStream_t to enqueue on.
 * Malformed offsets give wrong results but never an out-of-bounds access
 * (they are clamped as in wkv7_fwd_varlen, and the checkpoint storage is
 * bounded).  Output buffers must not overlap any input or each other.
 */
wkv7_status_t wkv7_bwd_varlen(int dtype, int N, int total_T, int H, int K, int V,
                              const int32_t *cu_seqlens,
                              const void *r, const void *w, const void *k,
                              const void *v, const void *a, const void *b,
                              const float *initial_state, int n_state, const int32_t *state_map,
                              const uint8_t *mask, const void *d_o, const float *d_final_state,
                              void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                              float *d_initial_state, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Workspace bytes wkv7_bwd_varlen needs: two fp32 K x V states per head for
 * each of ceil(total_T/16) + N chunks (a bound on the sequences' chunk
 * count), then N + 1 int32 chunk offsets; 0 for arguments wkv7_bwd_varlen
 * would reject. */
size_t wkv7_bwd_varlen_workspace_bytes(int N, int total_T, int H, int K, int V);

/*
 * wkv7_gdn_bwd -- gradients of wkv7_gdn_fwd (fixed-length form) for the
 * upstream gradients of every output and of the final state (rwkv-ops
 * README, sections "gdn_recurrent 使用方法" and "gdn_chunk 使用方法": the
 * training entries gated_delta_net_recurrent and gated_delta_net_chunk
 * backpropagate; same reading of the update as wkv7_gdn_fwd).
 *
 *   dtype          WKV7_F32 or WKV7_BF16 for q,k,v,g,beta, d_o and the five
 *                  input gradients.  All arithmetic is fp32.
 *   B, T, H, K, V  as for wkv7_gdn_fwd; T >= 0.
 *   q,k,v,g,beta   exactly the forward's inputs.  Read only.
 *   initial_state  [n_state,H,K,V] fp32 (n_state 1: one state shared by all
 *                  B sequences) or NULL (zeros).  Read only.
 *   n_state        1 or B when initial_state is given; ignored otherwise.
 *   d_o            [B,T,H,V] dtype.  Read only.
 *   d_final_state  [B,H,K,V] fp32 or NULL (zero).  Read only.
 *   dq, dk         [B,T,H,K] dtype; dv [B,T,H,V] dtype; dg, dbeta [B,T,H]
 *                  dtype.  Written (every element).
 *   d_initial_state [n_state,H,K,V] fp32 ([B,H,K,V] without initial_state:
 *                  the gradient of the zero start) or NULL (not written).
 *                  With a shared state it is the sum over the B sequences.
 *   workspace      DEVICE buffer of at least wkv7_gdn_bwd_workspace_bytes(...)
 *                  bytes, 16-byte aligned, owned by the caller; contents on
 *                  entry are ignored and on return are unspecified.  May be
 *                  NULL when T == 0.
 *   stream         hipStream_t to enqueue on.
 * Output buffers must not overlap any input or each other.  With T == 0,
 * d_initial_state receives d_final_state (summed over B for a shared state;
 * zeros when NULL).
 */
wkv7_status_t wkv7_gdn_bwd(int dtype, int B, int T, int H, int K, int V,
                           const void *q, const void *k, const void *v,
                           const void *g, const void *beta,
                           const float *initial_state, int n_state,
                           const void *d_o, const float *d_final_state,
                           void *dq, void *dk, void *dv, void *dg, void *dbeta,
                           float *d_initial_state, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Workspace bytes wkv7_gdn_bwd needs: two fp32 [B,H,K,V] state sets (each
 * rounded up to 256 bytes) and the workspace of wkv7_bwd at the same sizes;
 * 0 for arguments wkv7_gdn_bwd would reject. */
size_t wkv7_gdn_bwd_workspace_bytes(int B, int T, int H, int K, int V);

/*
 * wkv7_gdn_bwd_varlen -- gradients of wkv7_gdn_fwd_varlen (N packed Gated
 * DeltaNet sequences; same reading of the update as wkv7_gdn_fwd).  Sequence
 * n gets exactly the gradients wkv7_gdn_bwd gives for that one sequence.
 *
 *   dtype, N, total_T, H, K, V, cu_seqlens, q,k,v,g,beta, initial_state,
 *   n_state, state_map
 *                  as for wkv7_gdn_fwd_varlen (g and beta are [total_T,H];
 *                  without a map the pool has N rows or one row shared by
 *                  every sequence).  Read only.
 *   d_o            [total_T,H,V] dtype.  Read only.
 *   d_final_state  [N,H,K,V] fp32 or NULL (zero).  Read only.
 *   dq, dk         [total_T,H,K] dtype; dv [total_T,H,V]; dg, dbeta
 *                  [total_T,H].  Written at every token of every sequence.
 *   d_initial_state [N,H,K,V] fp32 or NULL: row n is the gradient of the
 *                  state sequence n started from (rows of sequences that
 *                  share a pool entry are the caller's to add).  Written.
 *   workspace      DEVICE buffer of at least
 *                  wkv7_gdn_bwd_varlen_workspace_bytes(...) bytes, 16-byte
 *                  aligned, owned by the caller.  May be NULL when
 *                  total_T == 0.
 *   stream         hipStream_t to enqueue on.
 */
wkv7_status_t wkv7_gdn_bwd_varlen(int dtype, int N, int total_T, int H, int K, int V,
                                  const int32_t *cu_seqlens,
                                  const void *q, const void *k, const void *v,
                                  const void *g, const void *beta,
                                  const float *initial_state, int n_state, const int32_t *state_map,
                                  const void *d_o, const float *d_final_state,
                                  void *dq, void *dk, void *dv, void *dg, void *dbeta,
                                  float *d_initial_state, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Workspace bytes wkv7_gdn_bwd_varlen needs (the same as
 * wkv7_bwd_varlen_workspace_bytes). */
size_t wkv7_gdn_bwd_varlen_workspace_bytes(int N, int total_T, int H, int K, int V);

/*
 * wkv7_step -- one decode token per sequence, state updated in place
 * (section "rwkv7_op_rnn 使用方法": the T = 1 case of the forward).
 *
 *   dtype          WKV7_F32 or WKV7_BF16 for r,w,k,v,a,b and o.
 *   B, H, K, V     as for wkv7_fwd; B, H >= 1; K == V in {64, 128}.
 *   r,w,k,a,b      [B,H,K] dtype.  Read only.
 *   v              [B,H,V] dtype.  Read only.
 *   state          [B,H,K,V] fp32.  Read, then overwritten with the new state.
 *   o              [B,H,V] dtype.  Written.  Must not overlap state.
 *   stream         hipStream_t to enqueue on.
 */
wkv7_status_t wkv7_step(int dtype, int B, int H, int K, int V,
                        const void *r, const void *w, const void *k,
                        const void *v, const void *a, const void *b,
                        float *state, void *o, void *stream);

/*
 * wkv7_gdn_step -- one Gated DeltaNet decode token per sequence (rwkv-ops
 * README, section "gdn_recurrent 使用方法", gated_delta_net_recurrent_single_step:
 * the T = 1 case of wkv7_gdn_fwd, with the same reading of the update).
 *
 *   dtype          WKV7_F32 or WKV7_BF16 for q,k,v,g,beta and o.
 *   B, H, K, V     as for wkv7_step.
 *   q, k           [B,H,K] dtype, raw (normalised inside).  Read only.
 *   v              [B,H,V] dtype.  Read only.
 *   g, beta        [B,H] dtype.  Read only.
 *   state_in       [n_state,H,K,V] fp32 with n_state 1 (shared) or B, or NULL
 *                  for a zero state.  Read only.
 *   n_state        1 or B when state_in is given.
 *   state_out      [B,H,K,V] fp32.  Written with the next state.  May be the
 *                  same buffer as state_in when n_state == B (or B == 1): an
 *                  in-place update.
 *   o              [B,H,V] dtype.  Written.  Must not overlap a state.
 *   stream         hipStream_t to enqueue on.
 */
wkv7_status_t wkv7_gdn_step(int dtype, int B, int H, int K, int V,
                            const void *q, const void *k, const void *v,
                            const void *g, const void *beta,
                            const float *state_in, int n_state, float *state_out,
                            void *o, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *wkv7_strerror(int status);

/* Which kernel wkv7_fwd would launch for these arguments under algo:
 * returns WKV7_ALGO_RECURRENT or WKV7_ALGO_CHUNKED, or -1 if the arguments
 * would be rejected.  Host only; launches nothing. */
int wkv7_fwd_path(int dtype, int B, int T, int H, int K, int V, int algo);

/* Bytes of the device array that backs wkv7_bwd_noalloc's scratch, one
 * array per GPU, held from the first call on that GPU until the process
 * ends. */
#define WKV7_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * wkv7_bwd_noalloc -- wkv7_bwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight training loops, harnesses that
 * forbid hipMalloc.  It computes exactly what wkv7_bwd computes (the same
 * kernels), with the same arguments minus the workspace: the backward's
 * scratch (state checkpoints, per-sequence gradients of a shared initial
 * state) lives in a fixed device array of WKV7_NOALLOC_SCRATCH_BYTES bytes
 * inside the library instead.  The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.  Its first call on a GPU looks up
 * that GPU's copy of the array (with that GPU current); later calls reuse it.
 *
 *   arguments      as for wkv7_bwd, without workspace / workspace_bytes.
 * Returns WKV7_ERR_TOO_LARGE when wkv7_bwd_workspace_bytes(B,T,H,K,V)
 * exceeds WKV7_NOALLOC_SCRATCH_BYTES, that is when B H (2 ceil(T/16) + 1)
 * exceeds 4096 at K = V = 64 or 1024 at K = V = 128 (for example one
 * sequence of 8 heads up to T = 4080 at 64), after the same argument checks
 * as wkv7_bwd.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (the backward reads nothing of it that it has not written in the
 * same call, so nothing needs clearing): calls that overlap in time on one
 * GPU, on different streams, race on it and must be serialised by the
 * caller.
 */
wkv7_status_t wkv7_bwd_noalloc(int dtype, int B, int T, int H, int K, int V,
                               const void *r, const void *w, const void *k,
                               const void *v, const void *a, const void *b,
                               const float *initial_state, int n_state, const uint8_t *mask,
                               const void *d_o, const float *d_final_state,
                               void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                               float *d_initial_state, void *stream);

/*
 * wkv7_set_wait_limit -- test hook for the failure path of the chunked
 * forward.  Its producer and consumer waves hand chunks over through
 * counters in on-chip memory, and every wait on a counter is bounded: after
 * `polls` polls (default 2^20, about 30 ms) the wave gives up rather than
 * hang the GPU.  A give-up is made visible in the results: the affected
 * sequence's state becomes NaN, so the output rows of the chunk being
 * processed, every later output and its final_state are NaN.
 *
 *   polls   new limit for launches made after this call: 0 gives up at once
 *           (every wait fails, so every chunked output is NaN), a negative
 *           value restores the default.
 * Returns the previous limit.  This is the one piece of mutable state in
 * the library (process-wide, read at each chunked launch); it is meant for
 * tests that force the give-up from the host, and normal use never calls it.
 */
int wkv7_set_wait_limit(int polls);

/* ABI version of this header (major * 100 + minor): 200 adds n_state (a
 * broadcast initial state) to wkv7_fwd and wkv7_bwd, accepts a one-row pool
 * without state_map in wkv7_fwd_varlen and wkv7_bwd_varlen, and adds
 * wkv7_set_wait_limit; 201 adds wkv7_bwd_noalloc; earlier: 101 adds wkv7_fwd_varlen,
 * 102 adds wkv7_gdn_fwd, 103 adds wkv7_bwd and wkv7_bwd_workspace_bytes,
 * 104 adds wkv7_gdn_step, 105 adds wkv7_gdn_fwd_varlen, 106 adds wkv7_gdn_bwd and
 * wkv7_gdn_bwd_workspace_bytes, 107 adds wkv7_bwd_varlen and
 * wkv7_bwd_varlen_workspace_bytes, 108 adds wkv7_gdn_bwd_varlen and
 * wkv7_gdn_bwd_varlen_workspace_bytes. */
int wkv7_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_H */

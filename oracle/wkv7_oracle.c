/*
 * wkv7_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential fp64 CPU evaluation of the RWKV-7 WKV7
 * generalized-delta-rule forward recurrence.  It exists so that the HIP
 * kernels can be checked against something obviously correct.  Only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it; the product path never calls it and shares no code with it.
 *
 * What it computes (per sequence b and head h, independently):
 *
 *   S      : K x V state, starts at initial_state[b,h] (zeros when absent)
 *   for t = 0 .. T-1:
 *     if mask[b,t] != 0 (or no mask):
 *       sb[j]   = sum_i b_t[i] * S[i][j]                       (old state)
 *       S[i][j] = exp(w_t[i]) * S[i][j] + a_t[i] * sb[j] + k_t[i] * v_t[j]
 *     o_t[j] = sum_i r_t[i] * S[i][j]                          (new state)
 *   final_state[b,h] = S
 *
 * Sources (rwkv-ops README, PyPI page rwkv-ops 0.7.4 and the rwkv_ops 0.9.0
 * wheel METADATA, section "rwkv7op 使用方法", docstring of
 * generalized_delta_rule):
 *   - r, w, k, a, b are [B,T,H,K], v and o are [B,T,H,V], seq-first layout;
 *   - w ("gk") is the decay in log space, so the per-channel factor is exp(w);
 *   - mask [B,T]: 1 updates the state, 0 leaves it unchanged;
 *   - initial_state / final_state are [N,H,K,V] with N = number of sequences,
 *     and a missing initial state means zeros (section "rwkv7_op_rnn 使用方法"
 *     states the same for the single-step operator).
 * The pages do not print the update equation itself.  The reading used here
 * is the generalized delta rule written above: the low-rank term a_t (b_t^T S)
 * acts on the state before this token's decay, a sits on the K side, b
 * contracts with the state, and o_t reads the updated state S_t, with no
 * scale on r and no bonus term.  A masked token keeps S and still emits
 * o_t = S^T r_t.
 *
 * Layouts (row-major, C order):
 *   r,w,k,a,b : [B][T][H][K]     v, o : [B][T][H][V]
 *   state     : [B][H][K][V]     mask : [B][T] uint8
 *
 * Parity pins (closed forms, invariants, hand-worked examples, finite
 * differences) live in tests/test_oracle_pins.py (forward and step),
 * tests/test_oracle_bwd_pins.py (backward), tests/test_oracle_gdn_pins.py
 * (Gated DeltaNet forward) and tests/test_oracle_gdn_bwd_pins.py (Gated
 * DeltaNet backward); every function here is pinned by them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX_TOK(b, t, h, i, T, H, D) ((((size_t)(b) * (T) + (t)) * (H) + (h)) * (D) + (i))
#define IDX_ST(b, h, i, j, H, K, V) ((((size_t)(b) * (H) + (h)) * (K) + (i)) * (V) + (j))

/* One token of the recurrence on a single K x V state (row-major, in place).
 * sb is caller scratch of length V. */
static void one_token(int K, int V, double *S, const double *r, const double *w,
                      const double *k, const double *v, const double *a,
                      const double *b, int update, double *o, double *sb)
{
    if (update) {
        for (int j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int i = 0; i < K; ++i) acc += b[i] * S[(size_t)i * V + j];
            sb[j] = acc;
        }
        for (int i = 0; i < K; ++i) {
            double d = exp(w[i]);
            for (int j = 0; j < V; ++j) {
                double *s = &S[(size_t)i * V + j];
                *s = d * (*s) + a[i] * sb[j] + k[i] * v[j];
            }
        }
    }
    for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += r[i] * S[(size_t)i * V + j];
        o[j] = acc;
    }
}

/* Forward over a whole sequence for every (b, h).
 * s0 may be NULL (zeros), mask may be NULL (all tokens update),
 * s_final may be NULL (not written).  s_final may alias s0.
 * Returns 0, or -1 on bad sizes / missing buffers. */
int wkv7_oracle_fwd(int B, int T, int H, int K, int V,
                    const double *r, const double *w, const double *k,
                    const double *v, const double *a, const double *b,
                    const double *s0, const uint8_t *mask,
                    double *o, double *s_final)
{
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return -1;
    if (T > 0 && (!r || !w || !k || !v || !a || !b || !o)) return -1;
    const long long nseq = (long long)B * H;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < nseq; ++bh) {
        const int bb = (int)(bh / H), h = (int)(bh % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)K * V);
        double *sb = (double *)malloc(sizeof(double) * (size_t)V);
        if (s0)
            memcpy(S, &s0[IDX_ST(bb, h, 0, 0, H, K, V)], sizeof(double) * (size_t)K * V);
        else
            memset(S, 0, sizeof(double) * (size_t)K * V);
        for (int t = 0; t < T; ++t) {
            const int upd = mask ? (mask[(size_t)bb * T + t] != 0) : 1;
            one_token(K, V, S,
                      &r[IDX_TOK(bb, t, h, 0, T, H, K)], &w[IDX_TOK(bb, t, h, 0, T, H, K)],
                      &k[IDX_TOK(bb, t, h, 0, T, H, K)], &v[IDX_TOK(bb, t, h, 0, T, H, V)],
                      &a[IDX_TOK(bb, t, h, 0, T, H, K)], &b[IDX_TOK(bb, t, h, 0, T, H, K)],
                      upd, &o[IDX_TOK(bb, t, h, 0, T, H, V)], sb);
        }
        if (s_final)
            memcpy(&s_final[IDX_ST(bb, h, 0, 0, H, K, V)], S, sizeof(double) * (size_t)K * V);
        free(sb);
        free(S);
    }
    return 0;
}

/* Single-token decode for every (b, h): inputs are [B][H][K] ([B][H][V] for
 * v and o); state [B][H][K][V] is read and overwritten in place.  This is
 * the T = 1 case of the forward (section "rwkv7_op_rnn 使用方法": the
 * single-step operator reuses the rwkv7_op definition). */
int wkv7_oracle_step(int B, int H, int K, int V,
                     const double *r, const double *w, const double *k,
                     const double *v, const double *a, const double *b,
                     double *state, double *o)
{
    if (B < 0 || H < 0 || K <= 0 || V <= 0) return -1;
    if ((long long)B * H > 0 && (!r || !w || !k || !v || !a || !b || !state || !o)) return -1;
    const long long nseq = (long long)B * H;

#pragma omp parallel for schedule(static)
    for (long long bh = 0; bh < nseq; ++bh) {
        double *sb = (double *)malloc(sizeof(double) * (size_t)V);
        one_token(K, V, &state[(size_t)bh * K * V],
                  &r[(size_t)bh * K], &w[(size_t)bh * K], &k[(size_t)bh * K],
                  &v[(size_t)bh * V], &a[(size_t)bh * K], &b[(size_t)bh * K],
                  1, &o[(size_t)bh * V], sb);
        free(sb);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Backward of the forward above: the reverse-mode derivative of the same
 * recurrence (the rwkv-ops README lists generalized_delta_rule as the
 * trainable entry, section "rwkv7op 使用方法"; the derivative itself is not
 * on the pages and follows from the recurrence by the chain rule).
 *
 * Given d_o = dL/do [B][T][H][V] and d_sf = dL/dS_T [B][H][K][V] (NULL for
 * zero), it returns dL/d{r,w,k,v,a,b} and dL/dS_0.  With S_{t-1} the state
 * before token t and S_t the state after it:
 *
 *   dS  <- d_sf
 *   for t = T-1 .. 0:
 *     dS     += r_t d_o_t^T                      (o_t = S_t^T r_t)
 *     dr_t    = S_t d_o_t
 *     if token t updates:
 *       sb      = S_{t-1}^T b_t,   ad = dS^T a_t
 *       dk_t    = dS v_t,          dv_t = dS^T k_t
 *       da_t    = dS sb,           db_t = S_{t-1} ad
 *       dw_t[i] = exp(w_t[i]) sum_j dS[i][j] S_{t-1}[i][j]
 *       dS      = diag(exp(w_t)) dS + b_t ad^T   (dL/dS_{t-1})
 *     else: dw, dk, dv, da, db of token t are 0 and dS passes through
 *   d_s0 = dS
 *
 * Every state S_0 .. S_T of a sequence is kept (T+1 K x V fp64 matrices per
 * sequence), so memory grows with T.  d_s0 may be NULL. */
int wkv7_oracle_bwd(int B, int T, int H, int K, int V,
                    const double *r, const double *w, const double *k,
                    const double *v, const double *a, const double *b,
                    const double *s0, const uint8_t *mask,
                    const double *d_o, const double *d_sf,
                    double *dr, double *dw, double *dk, double *dv,
                    double *da, double *db, double *d_s0)
{
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return -1;
    if (T > 0 && (!r || !w || !k || !v || !a || !b || !d_o || !dr || !dw || !dk || !dv || !da || !db))
        return -1;
    const long long nseq = (long long)B * H;
    const size_t KV = (size_t)K * V;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < nseq; ++bh) {
        const int bb = (int)(bh / H), h = (int)(bh % H);
        double *S = (double *)malloc(sizeof(double) * KV * ((size_t)T + 1));
        double *dS = (double *)malloc(sizeof(double) * KV);
        double *vec = (double *)malloc(sizeof(double) * (size_t)(V > K ? V : K) * 2);
        if (!S || !dS || !vec) {
            failed = 1;
            free(S); free(dS); free(vec);
            continue;
        }
        double *sb = vec, *ad = vec + (V > K ? V : K);
        /* forward, keeping every state: S + t*KV is S_t */
        if (s0)
            memcpy(S, &s0[IDX_ST(bb, h, 0, 0, H, K, V)], sizeof(double) * KV);
        else
            memset(S, 0, sizeof(double) * KV);
        for (int t = 0; t < T; ++t) {
            const int upd = mask ? (mask[(size_t)bb * T + t] != 0) : 1;
            memcpy(S + (size_t)(t + 1) * KV, S + (size_t)t * KV, sizeof(double) * KV);
            double *o_unused = sb;   /* the forward's output is not needed here */
            one_token(K, V, S + (size_t)(t + 1) * KV,
                      &r[IDX_TOK(bb, t, h, 0, T, H, K)], &w[IDX_TOK(bb, t, h, 0, T, H, K)],
                      &k[IDX_TOK(bb, t, h, 0, T, H, K)], &v[IDX_TOK(bb, t, h, 0, T, H, V)],
                      &a[IDX_TOK(bb, t, h, 0, T, H, K)], &b[IDX_TOK(bb, t, h, 0, T, H, K)],
                      upd, o_unused, ad);
        }
        /* reverse */
        if (d_sf)
            memcpy(dS, &d_sf[IDX_ST(bb, h, 0, 0, H, K, V)], sizeof(double) * KV);
        else
            memset(dS, 0, sizeof(double) * KV);
        for (int t = T - 1; t >= 0; --t) {
            const int upd = mask ? (mask[(size_t)bb * T + t] != 0) : 1;
            const double *St = S + (size_t)(t + 1) * KV, *Sp = S + (size_t)t * KV;
            const double *rt = &r[IDX_TOK(bb, t, h, 0, T, H, K)], *wt = &w[IDX_TOK(bb, t, h, 0, T, H, K)];
            const double *kt = &k[IDX_TOK(bb, t, h, 0, T, H, K)], *vt = &v[IDX_TOK(bb, t, h, 0, T, H, V)];
            const double *at = &a[IDX_TOK(bb, t, h, 0, T, H, K)], *bt = &b[IDX_TOK(bb, t, h, 0, T, H, K)];
            const double *dot = &d_o[IDX_TOK(bb, t, h, 0, T, H, V)];
            double *drt = &dr[IDX_TOK(bb, t, h, 0, T, H, K)], *dwt = &dw[IDX_TOK(bb, t, h, 0, T, H, K)];
            double *dkt = &dk[IDX_TOK(bb, t, h, 0, T, H, K)], *dvt = &dv[IDX_TOK(bb, t, h, 0, T, H, V)];
            double *dat = &da[IDX_TOK(bb, t, h, 0, T, H, K)], *dbt = &db[IDX_TOK(bb, t, h, 0, T, H, K)];
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j) dS[(size_t)i * V + j] += rt[i] * dot[j];
            for (int i = 0; i < K; ++i) {
                double acc = 0.0;
                for (int j = 0; j < V; ++j) acc += St[(size_t)i * V + j] * dot[j];
                drt[i] = acc;
            }
            if (!upd) {
                for (int i = 0; i < K; ++i) dwt[i] = dkt[i] = dat[i] = dbt[i] = 0.0;
                for (int j = 0; j < V; ++j) dvt[j] = 0.0;
                continue;
            }
            for (int j = 0; j < V; ++j) {
                double s1 = 0.0, s2 = 0.0, s3 = 0.0;
                for (int i = 0; i < K; ++i) {
                    s1 += bt[i] * Sp[(size_t)i * V + j];
                    s2 += at[i] * dS[(size_t)i * V + j];
                    s3 += kt[i] * dS[(size_t)i * V + j];
                }
                sb[j] = s1;
                ad[j] = s2;
                dvt[j] = s3;
            }
            for (int i = 0; i < K; ++i) {
                double ck = 0.0, ca = 0.0, cb = 0.0, cw = 0.0;
                for (int j = 0; j < V; ++j) {
                    const double g = dS[(size_t)i * V + j], sp = Sp[(size_t)i * V + j];
                    ck += g * vt[j];
                    ca += g * sb[j];
                    cb += sp * ad[j];
                    cw += g * sp;
                }
                dkt[i] = ck;
                dat[i] = ca;
                dbt[i] = cb;
                dwt[i] = exp(wt[i]) * cw;
            }
            for (int i = 0; i < K; ++i) {
                const double d = exp(wt[i]);
                for (int j = 0; j < V; ++j) dS[(size_t)i * V + j] = d * dS[(size_t)i * V + j] + bt[i] * ad[j];
            }
        }
        if (d_s0) memcpy(&d_s0[IDX_ST(bb, h, 0, 0, H, K, V)], dS, sizeof(double) * KV);
        free(vec);
        free(dS);
        free(S);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------
 * Gated DeltaNet forward (rwkv-ops README, section "gdn_recurrent 使用方法",
 * interface of gated_delta_net_recurrent; the same interface is listed for
 * the chunkwise gated_delta_net_chunk).  The page fixes the interface:
 *   q, k [B,T,H,K] are L2-normalised inside the operator; v [B,T,H,V];
 *   g [B,T,H] is a log-space decay gate; beta [B,T,H] is a write strength
 *   already passed through a sigmoid (in (0,1)); initial_state is [B,H,K,V]
 *   or [1,H,K,V] (shared); out has v's shape.
 * It does not print the recurrence.  The reading used is the textbook gated
 * delta rule with a K x V state:
 *
 *   qn = q / sqrt(sum q^2 + eps),  kn = k / sqrt(sum k^2 + eps),  eps = 1e-6
 *   S  = exp(g) * (I - beta kn kn^T) S  +  beta kn v^T
 *   o  = S^T qn
 *
 * (no scale on q).  n_s0 is 1 (one shared initial state) or B.
 * ------------------------------------------------------------------------ */
int gdn_oracle_fwd(int B, int T, int H, int K, int V,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta,
                   const double *s0, int n_s0, double *o, double *s_final)
{
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return -1;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    if (s0 && n_s0 != 1 && n_s0 != B) return -1;
    const double eps = 1e-6;
    const long long nseq = (long long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < nseq; ++bh) {
        const int bb = (int)(bh / H), h = (int)(bh % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)K * V);
        double *kS = (double *)malloc(sizeof(double) * (size_t)V);
        double *qn = (double *)malloc(sizeof(double) * (size_t)K);
        double *kn = (double *)malloc(sizeof(double) * (size_t)K);
        if (s0)
            memcpy(S, &s0[IDX_ST(n_s0 == 1 ? 0 : bb, h, 0, 0, H, K, V)], sizeof(double) * (size_t)K * V);
        else
            memset(S, 0, sizeof(double) * (size_t)K * V);
        for (int t = 0; t < T; ++t) {
            const double *qt = &q[IDX_TOK(bb, t, h, 0, T, H, K)];
            const double *kt = &k[IDX_TOK(bb, t, h, 0, T, H, K)];
            const double *vt = &v[IDX_TOK(bb, t, h, 0, T, H, V)];
            const double gt = g[((size_t)bb * T + t) * H + h];
            const double bt = beta[((size_t)bb * T + t) * H + h];
            double nq = 0.0, nk = 0.0;
            for (int i = 0; i < K; ++i) {
                nq += qt[i] * qt[i];
                nk += kt[i] * kt[i];
            }
            nq = 1.0 / sqrt(nq + eps);
            nk = 1.0 / sqrt(nk + eps);
            for (int i = 0; i < K; ++i) {
                qn[i] = qt[i] * nq;
                kn[i] = kt[i] * nk;
            }
            for (int j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i) acc += kn[i] * S[(size_t)i * V + j];
                kS[j] = acc;
            }
            const double alpha = exp(gt);
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j) {
                    double *s = &S[(size_t)i * V + j];
                    *s = alpha * (*s - bt * kn[i] * kS[j]) + bt * kn[i] * vt[j];
                }
            double *ot = &o[IDX_TOK(bb, t, h, 0, T, H, V)];
            for (int j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i) acc += qn[i] * S[(size_t)i * V + j];
                ot[j] = acc;
            }
        }
        if (s_final) memcpy(&s_final[IDX_ST(bb, h, 0, 0, H, K, V)], S, sizeof(double) * (size_t)K * V);
        free(kn);
        free(qn);
        free(kS);
        free(S);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Backward of gdn_oracle_fwd: the reverse-mode derivative of the same
 * recurrence (the pages list gated_delta_net_recurrent and
 * gated_delta_net_chunk as trainable entries).  For upstream gradients d_o
 * (of every output) and d_sf (of the final state, NULL = 0), walking the
 * tokens backwards with dS = dL/dS_t, P = S_{t-1}, alpha = exp(g_t),
 * y = P^T kn (the old state read at kn):
 *
 *   dS     += qn d_o_t^T
 *   dqn     = S_t d_o_t
 *   u       = dS^T kn
 *   dv_t    = beta u
 *   dbeta_t = sum_j u_j (v_j - alpha y_j)
 *   dg_t    = sum_ij dS_ij (S_t - beta kn v^T)_ij
 *   dkn     = beta dS v - alpha beta (dS y + P u)
 *   dS      = alpha (dS - beta kn u^T)               (dL/dS_{t-1})
 *
 * and through the normalisation x -> x s, s = 1/sqrt(sum x^2 + eps):
 *   dq = s (dqn - qn (qn . dqn)),  dk = s (dkn - kn (kn . dkn)).
 * d_s0 is [n_s0,H,K,V]: with one shared initial state (n_s0 = 1) it is the
 * sum over the B sequences; with no initial state it is the gradient of the
 * zero start, [B,H,K,V].  Every state S_0 .. S_T of a sequence is kept.
 * ------------------------------------------------------------------------ */
int gdn_oracle_bwd(int B, int T, int H, int K, int V,
                   const double *q, const double *k, const double *v,
                   const double *g, const double *beta,
                   const double *s0, int n_s0,
                   const double *d_o, const double *d_sf,
                   double *dq, double *dk, double *dv, double *dg, double *dbeta,
                   double *d_s0)
{
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return -1;
    if (T > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return -1;
    if (s0 && n_s0 != 1 && n_s0 != B) return -1;
    const double eps = 1e-6;
    const long long nseq = (long long)B * H;
    const size_t KV = (size_t)K * V;
    const int shared = s0 && n_s0 == 1;
    /* per-sequence initial-state gradients, summed afterwards when shared */
    double *ds_seq = NULL;
    if (d_s0 && shared) {
        ds_seq = (double *)calloc((size_t)nseq * KV, sizeof(double));
        if (!ds_seq && nseq > 0) return -2;
    }
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long bh = 0; bh < nseq; ++bh) {
        const int bb = (int)(bh / H), h = (int)(bh % H);
        const int KVmax = K > V ? K : V;
        double *S = (double *)malloc(sizeof(double) * KV * ((size_t)T + 1));
        double *dS = (double *)malloc(sizeof(double) * KV);
        double *vec = (double *)malloc(sizeof(double) * (size_t)KVmax * 6);
        if (!S || !dS || !vec) {
            failed = 1;
            free(S); free(dS); free(vec);
            continue;
        }
        double *qn = vec, *kn = vec + KVmax, *y = vec + 2 * KVmax, *u = vec + 3 * KVmax;
        double *dqn = vec + 4 * KVmax, *dkn = vec + 5 * KVmax;
        if (s0)
            memcpy(S, &s0[IDX_ST(shared ? 0 : bb, h, 0, 0, H, K, V)], sizeof(double) * KV);
        else
            memset(S, 0, sizeof(double) * KV);
        /* forward, keeping every state: S + t*KV is S_t */
        for (int t = 0; t < T; ++t) {
            const double *kt = &k[IDX_TOK(bb, t, h, 0, T, H, K)];
            const double *vt = &v[IDX_TOK(bb, t, h, 0, T, H, V)];
            const double gt = g[((size_t)bb * T + t) * H + h];
            const double bt = beta[((size_t)bb * T + t) * H + h];
            double nk = 0.0;
            for (int i = 0; i < K; ++i) nk += kt[i] * kt[i];
            nk = 1.0 / sqrt(nk + eps);
            for (int i = 0; i < K; ++i) kn[i] = kt[i] * nk;
            const double *P = S + (size_t)t * KV;
            double *Sn = S + (size_t)(t + 1) * KV;
            for (int j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i) acc += kn[i] * P[(size_t)i * V + j];
                y[j] = acc;
            }
            const double alpha = exp(gt);
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j)
                    Sn[(size_t)i * V + j] = alpha * (P[(size_t)i * V + j] - bt * kn[i] * y[j]) + bt * kn[i] * vt[j];
        }
        /* reverse */
        if (d_sf)
            memcpy(dS, &d_sf[IDX_ST(bb, h, 0, 0, H, K, V)], sizeof(double) * KV);
        else
            memset(dS, 0, sizeof(double) * KV);
        for (int t = T - 1; t >= 0; --t) {
            const double *qt = &q[IDX_TOK(bb, t, h, 0, T, H, K)];
            const double *kt = &k[IDX_TOK(bb, t, h, 0, T, H, K)];
            const double *vt = &v[IDX_TOK(bb, t, h, 0, T, H, V)];
            const double *dot = &d_o[IDX_TOK(bb, t, h, 0, T, H, V)];
            const size_t gi = ((size_t)bb * T + t) * H + h;
            const double gt = g[gi], bt = beta[gi], alpha = exp(gt);
            const double *P = S + (size_t)t * KV, *St = S + (size_t)(t + 1) * KV;
            double sq = 0.0, sk = 0.0;
            for (int i = 0; i < K; ++i) {
                sq += qt[i] * qt[i];
                sk += kt[i] * kt[i];
            }
            sq = 1.0 / sqrt(sq + eps);
            sk = 1.0 / sqrt(sk + eps);
            for (int i = 0; i < K; ++i) {
                qn[i] = qt[i] * sq;
                kn[i] = kt[i] * sk;
            }
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j) dS[(size_t)i * V + j] += qn[i] * dot[j];
            for (int i = 0; i < K; ++i) {
                double acc = 0.0;
                for (int j = 0; j < V; ++j) acc += St[(size_t)i * V + j] * dot[j];
                dqn[i] = acc;
            }
            for (int j = 0; j < V; ++j) {
                double ay = 0.0, au = 0.0;
                for (int i = 0; i < K; ++i) {
                    ay += kn[i] * P[(size_t)i * V + j];
                    au += kn[i] * dS[(size_t)i * V + j];
                }
                y[j] = ay;
                u[j] = au;
            }
            double db_acc = 0.0, dg_acc = 0.0;
            for (int j = 0; j < V; ++j) {
                dv[IDX_TOK(bb, t, h, j, T, H, V)] = bt * u[j];
                db_acc += u[j] * (vt[j] - alpha * y[j]);
            }
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j)
                    dg_acc += dS[(size_t)i * V + j] * (St[(size_t)i * V + j] - bt * kn[i] * vt[j]);
            dbeta[gi] = db_acc;
            dg[gi] = dg_acc;
            for (int i = 0; i < K; ++i) {
                double dsv = 0.0, dsy = 0.0, pu = 0.0;
                for (int j = 0; j < V; ++j) {
                    dsv += dS[(size_t)i * V + j] * vt[j];
                    dsy += dS[(size_t)i * V + j] * y[j];
                    pu += P[(size_t)i * V + j] * u[j];
                }
                dkn[i] = bt * dsv - alpha * bt * (dsy + pu);
            }
            double pq = 0.0, pk = 0.0;
            for (int i = 0; i < K; ++i) {
                pq += qn[i] * dqn[i];
                pk += kn[i] * dkn[i];
            }
            for (int i = 0; i < K; ++i) {
                dq[IDX_TOK(bb, t, h, i, T, H, K)] = sq * (dqn[i] - qn[i] * pq);
                dk[IDX_TOK(bb, t, h, i, T, H, K)] = sk * (dkn[i] - kn[i] * pk);
            }
            for (int i = 0; i < K; ++i)
                for (int j = 0; j < V; ++j)
                    dS[(size_t)i * V + j] = alpha * (dS[(size_t)i * V + j] - bt * kn[i] * u[j]);
        }
        if (d_s0) {
            double *dst = shared ? ds_seq + (size_t)bh * KV : &d_s0[IDX_ST(bb, h, 0, 0, H, K, V)];
            memcpy(dst, dS, sizeof(double) * KV);
        }
        free(vec);
        free(dS);
        free(S);
    }
    if (ds_seq) {
        /* shared initial state: sum the B sequences' gradients, in order */
        for (int h = 0; h < H; ++h)
            for (size_t e = 0; e < KV; ++e) {
                double acc = 0.0;
                for (int bb = 0; bb < B; ++bb) acc += ds_seq[((size_t)bb * H + h) * KV + e];
                d_s0[(size_t)h * KV + e] = acc;
            }
        free(ds_seq);
    }
    return failed ? -2 : 0;
}

/* Thread control for the OpenMP loop over (b, h); used to report how many
 * host threads a timed oracle run used. */
int wkv7_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void wkv7_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

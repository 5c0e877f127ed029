"""Pins for the fp64 oracle (CPU only).

The oracle is checked against results that the mathematics fixes without
re-typing its own loop: a hand-worked example, closed forms of special cases,
brute-force sums, transition-matrix products and invariants.  Each test notes
which plausible mistake in the oracle it would catch.

Operator source: rwkv-ops README, section "rwkv7op 使用方法" (interface,
log-space decay, mask semantics, [N,H,K,V] state) and section
"rwkv7_op_rnn 使用方法" (single-token operator with the same definition).
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "wkv7_handworked.txt")
TOL = 1e-10


def rand_inputs(rng, B, T, H, K, V, decay=True, lowrank=True, unit=True):
    r = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    k = rng.standard_normal((B, T, H, K))
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    w = -np.exp(rng.normal(-0.5, 0.5, (B, T, H, K))) if decay else np.zeros((B, T, H, K))
    if lowrank:
        kap = rng.standard_normal((B, T, H, K))
        kap /= np.linalg.norm(kap, axis=-1, keepdims=True)
        a = -kap
        b = kap * rng.random((B, T, H, K))
    else:
        a = np.zeros((B, T, H, K))
        b = np.zeros((B, T, H, K))
    return r, w, k, v, a, b


def close(x, y, tol=TOL):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    scale = max(1.0, float(np.max(np.abs(y))) if y.size else 1.0)
    assert x.shape == y.shape
    err = float(np.max(np.abs(x - y))) if x.size else 0.0
    assert err <= tol * scale, f"max abs err {err} (scale {scale})"


def load_golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            toks = rest.split()
            vals[key] = np.array([(-math.log(2.0) if t == "-ln2" else float(t)) for t in toks])
    return vals


# --- hand-worked example ---------------------------------------------------

@pytest.mark.parametrize("case", ["A", "B"])
def test_handworked_example(case):
    """Catches any error in the update order, the a/b roles, the decay factor
    exp(w), the mask and the post-update read-out, at exact small values."""
    g = load_golden()
    shp = (1, 3, 1, 2)
    r, w, k, v, a, b = (g[n].reshape(shp) for n in "rwkvab")
    mask = g["mask"].reshape(1, 3)
    s0 = g[case + ".s0"].reshape(1, 1, 2, 2)
    o, sf = oracle.fwd(r, w, k, v, a, b, s0, mask)
    close(o.reshape(-1), g[case + ".o"], 1e-12)
    close(sf.reshape(-1), g[case + ".final"], 1e-12)


# --- closed forms ----------------------------------------------------------

def test_p1_single_token_zero_state():
    """T=1 from a zero state: S_1 = k v^T and o = (k . r) v.  Catches reading
    the pre-update state, a scale on r, or a bonus term."""
    rng = np.random.default_rng(1)
    B, H, K, V = 3, 2, 5, 7
    r, w, k, v, a, b = rand_inputs(rng, B, 1, H, K, V)
    o, sf = oracle.fwd(r, w, k, v, a, b)
    kr = np.sum(k[:, 0] * r[:, 0], axis=-1)           # [B,H]
    close(o[:, 0], kr[..., None] * v[:, 0])
    close(sf, k[:, 0, :, :, None] * v[:, 0, :, None, :])


def test_p2_asymmetric_lowrank_sides():
    """w=0, k=0, S_0 = I, one token: S_1 = I + a b^T, so o(r=e_i) = e_i + a_i b.
    Catches swapping a and b, or applying the low-rank term on the wrong side."""
    rng = np.random.default_rng(2)
    K = 6
    B = K                                              # sequence i probes r = e_i
    a = rng.standard_normal((1, 1, 1, K)).repeat(B, 0)
    b = rng.standard_normal((1, 1, 1, K)).repeat(B, 0)
    r = np.eye(K).reshape(B, 1, 1, K)
    z = np.zeros((B, 1, 1, K))
    v = rng.standard_normal((B, 1, 1, K))
    s0 = np.broadcast_to(np.eye(K), (B, 1, K, K)).copy()
    o, sf = oracle.fwd(r, z, z, v, a, b, s0)
    expect_S = np.eye(K) + np.outer(a[0, 0, 0], b[0, 0, 0])
    for i in range(B):
        close(sf[i, 0], expect_S)
        close(o[i, 0, 0], np.eye(K)[i] + a[0, 0, 0, i] * b[0, 0, 0])


def test_p3_causal_linear_attention():
    """a = b = 0, w = 0: o_t = S_0^T r_t + sum_{j<=t} (k_j . r_t) v_j, by a
    brute-force double sum.  Catches causal off-by-one and layout mistakes."""
    rng = np.random.default_rng(3)
    B, T, H, K, V = 2, 9, 3, 4, 5
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V, decay=False, lowrank=False)
    s0 = rng.standard_normal((B, H, K, V))
    o, sf = oracle.fwd(r, w, k, v, a, b, s0)
    for bb in range(B):
        for h in range(H):
            for t in range(T):
                ref = np.zeros(V)
                for j in range(V):
                    acc = sum(r[bb, t, h, c] * s0[bb, h, c, j] for c in range(K))
                    for s in range(t + 1):
                        acc += sum(k[bb, s, h, c] * r[bb, t, h, c] for c in range(K)) * v[bb, s, h, j]
                    ref[j] = acc
                close(o[bb, t, h], ref)
            fin = s0[bb, h] + sum(np.outer(k[bb, s, h], v[bb, s, h]) for s in range(T))
            close(sf[bb, h], fin)


def test_p4_decay_product_sums():
    """a = b = 0, w != 0: per channel c, S_t[c,:] = exp(sum_{m<=t} w_m[c]) S_0[c,:]
    + sum_{j<=t} exp(sum_{j<m<=t} w_m[c]) k_j[c] v_j.  Catches exp(-w), a decay
    applied after the k v^T term, or a decay on the wrong axis."""
    rng = np.random.default_rng(4)
    B, T, H, K, V = 2, 11, 2, 5, 3
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V, decay=True, lowrank=False)
    s0 = rng.standard_normal((B, H, K, V))
    o, sf = oracle.fwd(r, w, k, v, a, b, s0)
    for bb in range(B):
        for h in range(H):
            for t in range(T):
                S = np.zeros((K, V))
                for c in range(K):
                    S[c] = math.exp(sum(w[bb, m, h, c] for m in range(t + 1))) * s0[bb, h, c]
                    for j in range(t + 1):
                        S[c] += math.exp(sum(w[bb, m, h, c] for m in range(j + 1, t + 1))) * k[bb, j, h, c] * v[bb, j, h]
                ref = np.array([sum(r[bb, t, h, c] * S[c, jj] for c in range(K)) for jj in range(V)])
                close(o[bb, t, h], ref)
                if t == T - 1:
                    close(sf[bb, h], S)


def test_p5_delta_rule_retrieval():
    """w = 0, a = -k, b = k, r = k with unit k: the delta rule overwrites the
    value stored under k, so o_t = v_t exactly whatever the history."""
    rng = np.random.default_rng(5)
    B, T, H, K = 2, 13, 2, 8
    kk = rng.standard_normal((B, T, H, K))
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, K))
    s0 = rng.standard_normal((B, H, K, K))
    o, _ = oracle.fwd(kk, np.zeros_like(kk), kk, v, -kk, kk, s0)
    close(o, v)


def test_p12_transition_matrix_product():
    """The recurrence is affine: S_t = A_t S_{t-1} + k_t v_t^T with
    A_t = diag(exp(w_t)) + a_t b_t^T.  Checked with explicit matrix products
    A_t ... A_1 S_0 + sum_j (A_t ... A_{j+1}) k_j v_j^T.  Catches a low-rank term
    computed from the decayed state, a/b swaps and w used without exp."""
    rng = np.random.default_rng(12)
    B, T, H, K, V = 2, 10, 2, 6, 4
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    o, sf = oracle.fwd(r, w, k, v, a, b, s0)
    for bb in range(B):
        for h in range(H):
            A = [np.diag(np.exp(w[bb, t, h])) + np.outer(a[bb, t, h], b[bb, t, h]) for t in range(T)]
            for t in range(T):
                P = np.eye(K)
                for s in range(t + 1):
                    P = A[s] @ P
                S = P @ s0[bb, h]
                for j in range(t + 1):
                    Pj = np.eye(K)
                    for s in range(j + 1, t + 1):
                        Pj = A[s] @ Pj
                    S = S + Pj @ np.outer(k[bb, j, h], v[bb, j, h])
                close(o[bb, t, h], S.T @ r[bb, t, h])
                if t == T - 1:
                    close(sf[bb, h], S)


# --- invariants ------------------------------------------------------------

def test_p6_all_masked_keeps_state():
    """mask = 0 everywhere: the final state equals the initial state bit for
    bit and o_t = S_0^T r_t."""
    rng = np.random.default_rng(6)
    B, T, H, K, V = 2, 7, 3, 4, 4
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    o, sf = oracle.fwd(r, w, k, v, a, b, s0, np.zeros((B, T), np.uint8))
    assert np.array_equal(sf, s0)
    close(o, np.einsum("bthc,bhcj->bthj", r, s0))


def test_p6_mask_equals_compacted_sequence():
    """A masked token is an identity step: running with a random mask equals
    running the sequence with the masked tokens removed, and a masked position
    reads the state left by the previous kept token.  Catches a mask that
    still decays, still adds k v^T, or is applied to the wrong sequence."""
    rng = np.random.default_rng(7)
    B, T, H, K, V = 3, 20, 2, 5, 4
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    mask = (rng.random((B, T)) < 0.6).astype(np.uint8)
    mask[1, :] = 0
    mask[2, :] = 1
    o, sf = oracle.fwd(r, w, k, v, a, b, s0, mask)
    for bb in range(B):
        keep = np.nonzero(mask[bb])[0]
        sl = lambda x: x[bb:bb + 1, keep]
        oc, sc = oracle.fwd(sl(r), sl(w), sl(k), sl(v), sl(a), sl(b), s0[bb:bb + 1])
        close(sf[bb], sc[0])
        close(o[bb, keep], oc[0])
        for t in np.nonzero(mask[bb] == 0)[0]:
            prev = keep[keep < t]
            if len(prev):
                j = np.searchsorted(keep, prev[-1]) + 1
                _, sp = oracle.fwd(*(x[bb:bb + 1, keep[:j]] for x in (r, w, k, v, a, b)), s0[bb:bb + 1])
                S = sp[0]
            else:
                S = s0[bb]
            close(o[bb, t], np.einsum("hc,hcj->hj", r[bb, t], S))


def test_p6_trailing_padding_equals_truncation():
    """Masking the last n tokens leaves the final state of the first T - n."""
    rng = np.random.default_rng(8)
    B, T, H, K, V = 2, 30, 2, 6, 6
    n = 3
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    mask = np.ones((B, T), np.uint8)
    mask[:, T - n:] = 0
    _, sf = oracle.fwd(r, w, k, v, a, b, s0, mask)
    _, st = oracle.fwd(*(x[:, :T - n] for x in (r, w, k, v, a, b)), s0)
    close(sf, st)


def test_p7_state_passing_composition():
    """fwd over [0,T) equals fwd over [T1,T) started from fwd([0,T1)).final,
    and the outputs concatenate."""
    rng = np.random.default_rng(9)
    B, T, H, K, V = 2, 25, 2, 5, 6
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    o, sf = oracle.fwd(r, w, k, v, a, b, s0)
    T1 = 11
    o1, s1 = oracle.fwd(*(x[:, :T1] for x in (r, w, k, v, a, b)), s0)
    o2, s2 = oracle.fwd(*(x[:, T1:] for x in (r, w, k, v, a, b)), s1)
    close(np.concatenate([o1, o2], axis=1), o)
    close(s2, sf)


def test_p8_linearity_in_state_and_values():
    """For fixed r, w, k, a, b the map (S_0, v) -> (o, S_T) is linear."""
    rng = np.random.default_rng(10)
    B, T, H, K, V = 1, 12, 2, 4, 3
    r, w, k, v1, a, b = rand_inputs(rng, B, T, H, K, V)
    v2 = rng.standard_normal(v1.shape)
    sA = rng.standard_normal((B, H, K, V))
    sB = rng.standard_normal((B, H, K, V))
    al, be = 0.7, -1.9
    o1, f1 = oracle.fwd(r, w, k, v1, a, b, sA)
    o2, f2 = oracle.fwd(r, w, k, v2, a, b, sB)
    o3, f3 = oracle.fwd(r, w, k, al * v1 + be * v2, a, b, al * sA + be * sB)
    close(o3, al * o1 + be * o2)
    close(f3, al * f1 + be * f2)


def test_p9_value_column_permutation():
    """Permuting the V columns of v and S_0 permutes o and S_T the same way."""
    rng = np.random.default_rng(11)
    B, T, H, K, V = 2, 9, 2, 4, 7
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    perm = rng.permutation(V)
    o, sf = oracle.fwd(r, w, k, v, a, b, s0)
    op, sp = oracle.fwd(r, w, k, v[..., perm], a, b, s0[..., perm])
    close(op, o[..., perm])
    close(sp, sf[..., perm])


def test_p10_step_loop_equals_forward():
    """Iterating the single-token operator T times equals the forward."""
    rng = np.random.default_rng(13)
    B, T, H, K, V = 2, 8, 3, 5, 5
    r, w, k, v, a, b = rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    o, sf = oracle.fwd(r, w, k, v, a, b, s0)
    S = s0
    for t in range(T):
        ot, S = oracle.step(r[:, t], w[:, t], k[:, t], v[:, t], a[:, t], b[:, t], S)
        close(ot, o[:, t])
    close(S, sf)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(14)
    B, H, K, V = 2, 3, 4, 4
    s0 = rng.standard_normal((B, H, K, V))
    z = np.zeros((B, 0, H, K))
    o, sf = oracle.fwd(z, z, z, z, z, z, s0)
    assert o.shape == (B, 0, H, V)
    assert np.array_equal(sf, s0)


def test_oracle_rejects_bad_sizes():
    lib = oracle._load()
    assert lib.wkv7_oracle_fwd(1, 1, 1, 0, 4, *([None] * 10)) == -1
    assert lib.wkv7_oracle_fwd(-1, 1, 1, 4, 4, *([None] * 10)) == -1
    assert lib.wkv7_oracle_step(1, 1, 4, 4, *([None] * 8)) == -1

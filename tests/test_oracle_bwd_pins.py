"""Pins of the fp64 backward oracle (oracle.bwd) to facts that do not come
from the backward itself:

  - central finite differences of L = sum(d_o * o) + sum(d_sf * S_T) through
    the forward oracle (itself pinned in test_oracle_pins.py), for every
    input element, with K != V and several (b, h) so that a transposed
    operand or a wrong index shows;
  - closed-form gradients of causal linear attention (a = b = 0, w = 0) and
    of pure decay (a = b = k = 0), by brute-force sums;
  - masked tokens: no gradient into w, k, v, a, b, and a sequence with
    masked tokens (and no output gradient there) has the gradients of its
    compacted version;
  - linearity in the upstream gradients; T = 0.

The derivative itself is not on the pages (the rwkv-ops README only lists
generalized_delta_rule as the trainable entry, section "rwkv7op 使用方法");
these pins tie it to the forward definition.
"""
import numpy as np
import pytest

import oracle

NAMES = ("r", "w", "k", "v", "a", "b")


def rand_inputs(rng, B, T, H, K, V, scale=0.6):
    x = {n: rng.standard_normal((B, T, H, V if n == "v" else K)) * scale for n in NAMES}
    x["w"] = -np.exp(rng.standard_normal((B, T, H, K)) * 0.5 - 0.7)
    x["w"][0, 1, 0, 0] = 0.2      # a positive log-decay is computed as written
    x["s0"] = rng.standard_normal((B, H, K, V)) * 0.5
    return x


def loss(x, mask, d_o, d_sf):
    o, sf = oracle.fwd(*(x[n] for n in NAMES), x["s0"], mask)
    return float(np.sum(d_o * o) + np.sum(d_sf * sf))


@pytest.mark.parametrize("masked", [False, True])
def test_finite_differences(masked):
    rng = np.random.default_rng(11 + masked)
    B, T, H, K, V = 2, 6, 2, 3, 2
    x = rand_inputs(rng, B, T, H, K, V)
    mask = None
    if masked:
        mask = np.ones((B, T), np.uint8)
        mask[0, 2] = 0
        mask[1, 0] = 0
        mask[1, 5] = 0
    d_o = rng.standard_normal((B, T, H, V))
    d_sf = rng.standard_normal((B, H, K, V))
    g = oracle.bwd(*(x[n] for n in NAMES), d_o, x["s0"], mask, d_sf)
    eps = 1e-6
    for name in NAMES + ("s0",):
        num = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = x[name][idx]
            x[name][idx] = keep + eps
            lp = loss(x, mask, d_o, d_sf)
            x[name][idx] = keep - eps
            lm = loss(x, mask, d_o, d_sf)
            x[name][idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, np.abs(num).max())
        np.testing.assert_allclose(g[name], num, rtol=0, atol=2e-7 * scale, err_msg=name)


def test_linear_attention_closed_form():
    """a = b = 0, w = 0: o_t = S0^T r_t + sum_{j<=t} (k_j . r_t) v_j and
    S_T = S0 + sum_j k_j v_j^T, so
      dr_t = S0 d_o_t + sum_{j<=t} (v_j . d_o_t) k_j
      dk_j = sum_{t>=j} (v_j . d_o_t) r_t + d_sf v_j
      dv_j = sum_{t>=j} (k_j . r_t) d_o_t + d_sf^T k_j
      ds0  = sum_t r_t d_o_t^T + d_sf."""
    rng = np.random.default_rng(3)
    T, K, V = 9, 4, 3
    r, k = rng.standard_normal((T, K)), rng.standard_normal((T, K))
    v = rng.standard_normal((T, V))
    s0 = rng.standard_normal((K, V))
    d_o, d_sf = rng.standard_normal((T, V)), rng.standard_normal((K, V))
    z = np.zeros((1, T, 1, K))
    g = oracle.bwd(r[None, :, None], z, k[None, :, None], v[None, :, None], z, z, d_o[None, :, None],
                   s0[None, None], None, d_sf[None, None])
    dr = np.array([s0 @ d_o[t] + sum((v[j] @ d_o[t]) * k[j] for j in range(t + 1)) for t in range(T)])
    dk = np.array([sum((v[j] @ d_o[t]) * r[t] for t in range(j, T)) + d_sf @ v[j] for j in range(T)])
    dv = np.array([sum((k[j] @ r[t]) * d_o[t] for t in range(j, T)) + d_sf.T @ k[j] for j in range(T)])
    ds0 = sum(np.outer(r[t], d_o[t]) for t in range(T)) + d_sf
    np.testing.assert_allclose(g["r"][0, :, 0], dr, atol=1e-12)
    np.testing.assert_allclose(g["k"][0, :, 0], dk, atol=1e-12)
    np.testing.assert_allclose(g["v"][0, :, 0], dv, atol=1e-12)
    np.testing.assert_allclose(g["s0"][0, 0], ds0, atol=1e-12)
    # b = 0 makes b^T S vanish and a = 0 makes a^T dS vanish: no gradient into a or b
    assert np.all(g["a"] == 0) and np.all(g["b"] == 0)


def test_pure_decay_closed_form():
    """a = b = k = 0: S_t = diag(e^{G_t}) S0 with G_t = sum_{m<=t} w_m, so
      dw_m[i] = sum_{t>=m} sum_j r_t[i] e^{G_t[i]} S0[i,j] d_o_t[j]
                + sum_j d_sf[i,j] e^{G_T[i]} S0[i,j]
      ds0[i,j] = sum_t e^{G_t[i]} r_t[i] d_o_t[j] + e^{G_T[i]} d_sf[i,j]."""
    rng = np.random.default_rng(4)
    T, K, V = 7, 3, 5
    r = rng.standard_normal((T, K))
    w = -np.exp(rng.standard_normal((T, K)) * 0.4 - 1.0)
    s0 = rng.standard_normal((K, V))
    d_o, d_sf = rng.standard_normal((T, V)), rng.standard_normal((K, V))
    z = np.zeros((1, T, 1, K))
    g = oracle.bwd(r[None, :, None], w[None, :, None], z, np.zeros((1, T, 1, V)), z, z,
                   d_o[None, :, None], s0[None, None], None, d_sf[None, None])
    G = np.cumsum(w, axis=0)
    dw = np.zeros((T, K))
    for m in range(T):
        for t in range(m, T):
            dw[m] += r[t] * np.exp(G[t]) * (s0 @ d_o[t])
        dw[m] += np.exp(G[-1]) * np.sum(d_sf * s0, axis=1)
    ds0 = sum(np.outer(np.exp(G[t]) * r[t], d_o[t]) for t in range(T)) + np.exp(G[-1])[:, None] * d_sf
    np.testing.assert_allclose(g["w"][0, :, 0], dw, atol=1e-12)
    np.testing.assert_allclose(g["s0"][0, 0], ds0, atol=1e-12)
    dr = np.array([np.exp(G[t]) * (s0 @ d_o[t]) for t in range(T)])
    np.testing.assert_allclose(g["r"][0, :, 0], dr, atol=1e-12)


def test_masked_tokens_match_compacted_sequence():
    """Masked tokens get no gradient into w, k, v, a, b.  With zero output
    gradient at the masked positions, the gradients of the kept tokens and of
    the initial state equal those of the sequence with the masked tokens
    removed."""
    rng = np.random.default_rng(5)
    T, H, K, V = 10, 1, 4, 4
    x = rand_inputs(rng, 1, T, H, K, V)
    mask = np.array([[1, 0, 1, 1, 0, 0, 1, 1, 0, 1]], np.uint8)
    keep = np.nonzero(mask[0])[0]
    d_o = rng.standard_normal((1, T, H, V))
    d_o[0, mask[0] == 0] = 0.0
    d_sf = rng.standard_normal((1, H, K, V))
    g = oracle.bwd(*(x[n] for n in NAMES), d_o, x["s0"], mask, d_sf)
    for n in ("w", "k", "v", "a", "b", "r"):
        assert np.all(g[n][0, mask[0] == 0] == 0.0), n
    gc = oracle.bwd(*(x[n][:, keep] for n in NAMES), d_o[:, keep], x["s0"], None, d_sf)
    for n in NAMES:
        np.testing.assert_allclose(g[n][:, keep], gc[n], atol=1e-12, err_msg=n)
    np.testing.assert_allclose(g["s0"], gc["s0"], atol=1e-12)


def test_masked_token_reads_previous_state():
    """o_t = S_{t-1}^T r_t at a masked token, so dr_t = S_{t-1} d_o_t."""
    rng = np.random.default_rng(6)
    T, K, V = 5, 3, 3
    x = rand_inputs(rng, 1, T, 1, K, V)
    mask = np.array([[1, 1, 0, 1, 1]], np.uint8)
    d_o = rng.standard_normal((1, T, 1, V))
    g = oracle.bwd(*(x[n] for n in NAMES), d_o, x["s0"], mask, None)
    _, s2 = oracle.fwd(*(x[n][:, :2] for n in NAMES), x["s0"], None)
    np.testing.assert_allclose(g["r"][0, 2, 0], s2[0, 0] @ d_o[0, 2, 0], atol=1e-12)


def test_linear_in_upstream_gradients():
    rng = np.random.default_rng(7)
    B, T, H, K, V = 2, 8, 2, 4, 3
    x = rand_inputs(rng, B, T, H, K, V)
    mask = (rng.random((B, T)) < 0.8).astype(np.uint8)
    do1, do2 = rng.standard_normal((2, B, T, H, V))
    sf1, sf2 = rng.standard_normal((2, B, H, K, V))
    g1 = oracle.bwd(*(x[n] for n in NAMES), do1, x["s0"], mask, sf1)
    g2 = oracle.bwd(*(x[n] for n in NAMES), do2, x["s0"], mask, sf2)
    g12 = oracle.bwd(*(x[n] for n in NAMES), do1 + 2 * do2, x["s0"], mask, sf1 + 2 * sf2)
    for n in NAMES + ("s0",):
        np.testing.assert_allclose(g12[n], g1[n] + 2 * g2[n], atol=1e-10, err_msg=n)


def test_empty_sequence_passes_state_gradient():
    rng = np.random.default_rng(8)
    K, V = 3, 4
    e = np.zeros((1, 0, 1, K))
    d_sf = rng.standard_normal((1, 1, K, V))
    g = oracle.bwd(e, e, e, np.zeros((1, 0, 1, V)), e, e, np.zeros((1, 0, 1, V)),
                   rng.standard_normal((1, 1, K, V)), None, d_sf)
    np.testing.assert_array_equal(g["s0"], d_sf)

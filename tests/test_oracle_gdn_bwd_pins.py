"""Pins of the fp64 Gated DeltaNet backward oracle (oracle.gdn_bwd) to facts
that do not come from the backward itself:

  - central finite differences of L = sum(d_o * o) + sum(d_sf * S_T) through
    the Gated DeltaNet forward oracle (itself pinned in
    test_oracle_gdn_pins.py), for every input element, with K != V, several
    (b, h), a per-sequence and a shared initial state;
  - the one-token closed form from a zero state, where S_1 = beta kn v^T and
    o = beta (kn . qn) v, worked by hand below;
  - scale invariance of the normalised inputs: q and k enter only through
    q/|q| and k/|k| (up to the 1e-6 in the norm), so their gradients are
    orthogonal to q and k;
  - beta = 0 (no writes): v and k get no gradient, and the output is the
    decayed initial state read at qn;
  - T = 0.

The pages give the interface and state that the training entries
(gated_delta_net_recurrent, gated_delta_net_chunk) backpropagate (rwkv-ops
README, sections "gdn_recurrent 使用方法" and "gdn_chunk 使用方法"); the
derivative is tied here to the forward definition.
"""
import numpy as np
import pytest

import oracle

EPS = 1e-6   # the norm's epsilon, sqrt(sum x^2 + 1e-6)


def rand_inputs(rng, B, T, H, K, V, n_s0):
    x = {"q": rng.standard_normal((B, T, H, K)), "k": rng.standard_normal((B, T, H, K)),
         "v": rng.standard_normal((B, T, H, V)) * 0.7,
         "g": -np.exp(rng.standard_normal((B, T, H)) * 0.5 - 1.0),
         "beta": 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))}
    x["s0"] = rng.standard_normal((n_s0, H, K, V)) * 0.5
    return x


def loss(x, d_o, d_sf):
    o, sf = oracle.gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"])
    return float(np.sum(d_o * o) + np.sum(d_sf * sf))


@pytest.mark.parametrize("n_s0", ["B", 1])
def test_finite_differences(n_s0):
    rng = np.random.default_rng(21 + (n_s0 == 1))
    B, T, H, K, V = 2, 5, 2, 3, 4
    x = rand_inputs(rng, B, T, H, K, V, B if n_s0 == "B" else 1)
    d_o = rng.standard_normal((B, T, H, V))
    d_sf = rng.standard_normal((B, H, K, V))
    g = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, x["s0"], d_sf)
    h = 1e-6
    for name in ("q", "k", "v", "g", "beta", "s0"):
        num = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = x[name][idx]
            x[name][idx] = keep + h
            lp = loss(x, d_o, d_sf)
            x[name][idx] = keep - h
            lm = loss(x, d_o, d_sf)
            x[name][idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, np.abs(num).max())
        np.testing.assert_allclose(g[name], num, rtol=0, atol=2e-7 * scale, err_msg=name)


def test_one_token_closed_form():
    """T = 1 from a zero state: S_1 = beta kn v^T, o = beta (kn . qn) v, so
    with c = kn . qn and e = v . d_o:
      dv = beta c d_o,  dbeta = c e,  dg = 0 (nothing to decay),
      dqn = beta e kn,  dkn = beta e qn (+ d_sf terms, here zero),
    and dq, dk are those projected off q, k and divided by the norms."""
    rng = np.random.default_rng(5)
    K, V = 5, 3
    q, k, v, do = rng.standard_normal(K), rng.standard_normal(K), rng.standard_normal(V), rng.standard_normal(V)
    beta, gg = 0.3, -0.4
    nq, nk = np.sqrt(q @ q + EPS), np.sqrt(k @ k + EPS)
    qn, kn = q / nq, k / nk
    c, e = kn @ qn, v @ do
    dqn, dkn = beta * e * kn, beta * e * qn
    want = {"v": beta * c * do, "beta": c * e, "g": 0.0,
            "q": (dqn - qn * (qn @ dqn)) / nq, "k": (dkn - kn * (kn @ dkn)) / nk}
    got = oracle.gdn_bwd(q[None, None, None], k[None, None, None], v[None, None, None],
                         np.full((1, 1, 1), gg), np.full((1, 1, 1), beta), do[None, None, None])
    for n in ("q", "k", "v"):
        np.testing.assert_allclose(got[n][0, 0, 0], want[n], rtol=1e-12, atol=1e-14, err_msg=n)
    np.testing.assert_allclose(got["beta"][0, 0, 0], want["beta"], rtol=1e-12)
    assert got["g"][0, 0, 0] == 0.0
    # the gradient of the zero initial state: dS_0 = e^g (dS_1 - beta kn u^T), dS_1 = qn d_o^T
    dS1 = np.outer(qn, do)
    u = dS1.T @ kn
    np.testing.assert_allclose(got["s0"][0, 0], np.exp(gg) * (dS1 - beta * np.outer(kn, u)), rtol=1e-12, atol=1e-15)


def test_normalised_inputs_are_scale_free():
    """o depends on q and k only through their directions (the 1e-6 in the
    norm aside), so dq . q = dk . k = 0 per token, up to that epsilon."""
    rng = np.random.default_rng(8)
    B, T, H, K, V = 1, 12, 2, 6, 5
    x = rand_inputs(rng, B, T, H, K, V, B)
    x["q"] *= 3.0
    x["k"] *= 3.0
    g = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], rng.standard_normal((B, T, H, V)), x["s0"])
    for n in ("q", "k"):
        dots = np.sum(g[n] * x[n], axis=-1)
        scale = np.abs(g[n]).max() * np.abs(x[n]).max()
        assert np.abs(dots).max() < 1e-6 * scale, n


def test_no_writes():
    """beta = 0: S_t = e^{G_t} S_0 and o_t = e^{G_t} S_0^T qn_t, so dv = dk =
    0, d_s0 = sum_t e^{G_t} qn_t d_o_t^T, dg_m = sum_{t>=m} e^{G_t} qn_t^T S_0
    d_o_t, and dbeta_t = sum_j u_j (v_j - e^{g_t} y_j) with the running dS."""
    rng = np.random.default_rng(9)
    T, K, V = 7, 4, 3
    x = rand_inputs(rng, 1, T, 1, K, V, 1)
    x["beta"][:] = 0.0
    d_o = rng.standard_normal((1, T, 1, V))
    g = oracle.gdn_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, x["s0"])
    assert np.all(g["v"] == 0.0) and np.all(g["k"] == 0.0)
    qn = x["q"][0, :, 0] / np.sqrt(np.sum(x["q"][0, :, 0] ** 2, axis=-1, keepdims=True) + EPS)
    G = np.cumsum(x["g"][0, :, 0])
    S0 = x["s0"][0, 0]
    ds0 = sum(np.exp(G[t]) * np.outer(qn[t], d_o[0, t, 0]) for t in range(T))
    np.testing.assert_allclose(g["s0"][0, 0], ds0, rtol=1e-12, atol=1e-14)
    per_t = np.array([np.exp(G[t]) * qn[t] @ S0 @ d_o[0, t, 0] for t in range(T)])
    dg = np.cumsum(per_t[::-1])[::-1]
    np.testing.assert_allclose(g["g"][0, :, 0], dg, rtol=1e-12, atol=1e-14)


def test_empty_sequence():
    rng = np.random.default_rng(10)
    B, H, K, V = 3, 2, 4, 4
    d_sf = rng.standard_normal((B, H, K, V))
    z = lambda *s: np.zeros(s)
    g = oracle.gdn_bwd(z(B, 0, H, K), z(B, 0, H, K), z(B, 0, H, V), z(B, 0, H), z(B, 0, H), z(B, 0, H, V),
                       rng.standard_normal((1, H, K, V)), d_sf)
    np.testing.assert_array_equal(g["s0"][0], d_sf.sum(axis=0))
    assert g["q"].shape == (B, 0, H, K)

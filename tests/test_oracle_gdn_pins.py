"""Pins of the fp64 Gated DeltaNet oracle (oracle.gdn_fwd) to facts that do
not come from the oracle itself.

The interface is the rwkv-ops README's (section "gdn_recurrent 使用方法"):
q, k L2-normalised inside, g a log-space decay gate, beta a write strength in
(0, 1).  The recurrence is the textbook gated delta rule
S = e^g (I - beta kn kn^T) S + beta kn v^T, o = S^T qn (see the oracle's C
header for this reading).
"""
import numpy as np
import pytest

import oracle

EPS = 1e-6


def unit(x):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + EPS)


def test_hand_worked_scalar_example():
    """K = V = 1, worked by hand: t0: alpha = 0.5, beta = 0.5, kn = +1,
    v = 4: S = 0.5 (1 - 0.5) 0 + 0.5 * 4 = 2, o = 2.  t1: alpha = 1,
    beta = 0.25, kn = -1, v = 8: S = (2 - 0.25 * 2) + 0.25 * (-1) * 8 = -0.5,
    o = -0.5 (qn = +1).  kn and qn differ from +-1 by the 1e-6 epsilon only."""
    q = np.array([1.0, 1.0]).reshape(1, 2, 1, 1)
    k = np.array([2.0, -3.0]).reshape(1, 2, 1, 1)
    v = np.array([4.0, 8.0]).reshape(1, 2, 1, 1)
    g = np.log(np.array([0.5, 1.0])).reshape(1, 2, 1)
    beta = np.array([0.5, 0.25]).reshape(1, 2, 1)
    o, sf = oracle.gdn_fwd(q, k, v, g, beta)
    assert np.allclose(o.ravel(), [2.0, -0.5], atol=1e-5)
    assert np.allclose(sf.ravel(), [-0.5], atol=1e-5)


def test_zero_beta_is_pure_decay():
    """beta = 0: S_t = e^{g_1 + .. + g_t} S_0 and o_t = S_t^T qn_t."""
    rng = np.random.default_rng(1)
    B, T, H, K, V = 2, 9, 2, 5, 3
    q, k = rng.standard_normal((2, B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = -rng.random((B, T, H))
    s0 = rng.standard_normal((B, H, K, V))
    o, sf = oracle.gdn_fwd(q, k, v, g, np.zeros((B, T, H)), s0)
    G = np.cumsum(g, axis=1)                           # [B,T,H]
    exp_o = np.einsum("bthk,bhkv->bthv", unit(q), s0) * np.exp(G)[..., None]
    assert np.allclose(o, exp_o, atol=1e-12)
    assert np.allclose(sf, s0 * np.exp(G[:, -1])[:, :, None, None], atol=1e-12)


def test_delta_rule_retrieval_and_overwrite():
    """g = 0, beta = 1, orthonormal keys: each write stores v under its key
    (o_t = v_t when q = k_t), and writing the same key again replaces the
    stored value instead of adding to it."""
    K = V = 4
    keys = np.eye(K)
    vals = np.arange(1.0, 1.0 + 5 * V).reshape(5, V)
    seq_k = np.stack([keys[0], keys[1], keys[2], keys[0], keys[3]])
    q = seq_k.copy()
    o, sf = oracle.gdn_fwd(q[None, :, None], seq_k[None, :, None], vals[None, :, None],
                           np.zeros((1, 5, 1)), np.ones((1, 5, 1)))
    o = o[0, :, 0]
    assert np.allclose(o, vals, atol=1e-5)
    # key 0 now holds the fourth value only
    assert np.allclose(sf[0, 0, 0], vals[3], atol=1e-5)


def test_scale_invariance_of_q_and_k():
    """q and k are normalised inside: positive rescaling changes nothing
    (up to the epsilon)."""
    rng = np.random.default_rng(2)
    B, T, H, K, V = 1, 12, 1, 6, 4
    q, k = rng.standard_normal((2, B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = -rng.random((B, T, H))
    beta = rng.random((B, T, H))
    o1, s1 = oracle.gdn_fwd(q, k, v, g, beta)
    o2, s2 = oracle.gdn_fwd(3.0 * q, 0.25 * k, v, g, beta)
    assert np.allclose(o1, o2, atol=1e-6) and np.allclose(s1, s2, atol=1e-6)


def test_shared_initial_state_broadcasts():
    rng = np.random.default_rng(3)
    B, T, H, K, V = 3, 5, 2, 4, 4
    q, k = rng.standard_normal((2, B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = -rng.random((B, T, H))
    beta = rng.random((B, T, H))
    s1 = rng.standard_normal((1, H, K, V))
    o1, f1 = oracle.gdn_fwd(q, k, v, g, beta, s1)
    o2, f2 = oracle.gdn_fwd(q, k, v, g, beta, np.repeat(s1, B, axis=0))
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("seed", [4, 5])
def test_matches_generalized_delta_rule_oracle_under_the_mapping(seed):
    """The gated delta rule is the generalized delta rule with w = g on every
    channel, a = -e^g beta kn, b = kn, k' = beta kn and r = qn; the two oracles
    are separate code, so their agreement pins both."""
    rng = np.random.default_rng(seed)
    B, T, H, K, V = 2, 23, 2, 8, 8
    q, k = rng.standard_normal((2, B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = -2.0 * rng.random((B, T, H))
    beta = rng.random((B, T, H))
    s0 = rng.standard_normal((B, H, K, V)) * 0.3
    o1, f1 = oracle.gdn_fwd(q, k, v, g, beta, s0)
    kn, qn = unit(k), unit(q)
    w = np.repeat(g[..., None], K, axis=-1)
    a = -(np.exp(g) * beta)[..., None] * kn
    kk = beta[..., None] * kn
    o2, f2 = oracle.fwd(qn, w, kk, v, a, kn, s0)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(f1, f2, atol=1e-12)

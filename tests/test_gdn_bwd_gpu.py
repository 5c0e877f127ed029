"""GPU parity of wkv7_gdn_bwd (gradients of the Gated DeltaNet forward)
against the fp64 Gated DeltaNet backward oracle, which is pinned to the
Gated DeltaNet forward by finite differences
(tests/test_oracle_gdn_bwd_pins.py).  The oracle differentiates the gated
delta rule directly; the GPU path maps it onto the WKV7 backward, so the two
share neither code nor the derivation.

Inputs follow the argument table of the rwkv-ops README, section
"gdn_recurrent 使用方法" (synth.make_gdn).  Tolerances, per gradient tensor:
the rules of the WKV7 backward (tests/test_bwd_gpu.py): bf16 I/O
|g - g_ref| <= 0.02 RMS(g_ref) + 2^-8 |g_ref|; fp32 I/O
|g - g_ref| <= 1e-4 RMS(g_ref) + 1e-5 |g_ref|; the initial-state gradient
(fp32 in both) by the fp32 rule.
"""
import numpy as np
import pytest

import harness as hz
import oracle
from rwkv_linear_attention_amd import synth, wkv7
from harness import check_grad

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")


def make_case(B, T, H, D, dtype, seed, init=True, n_state=None, dsf=True):
    inp = synth.make_gdn(B, T, H, D, seed=seed, dtype=dtype, init=init, n_state=n_state)
    rng = np.random.default_rng(seed + 11)
    d_o = synth.round_to(rng.standard_normal((B, T, H, D)).astype(np.float32), dtype)
    d_sf = (rng.standard_normal((B, H, D, D)) * 0.5).astype(np.float32) if dsf else None
    return inp, d_o, d_sf


def run_gpu(inp, d_o, d_sf, workspace=None):
    dt = inp["dtype"]
    dev = {n: synth.to_torch(inp[n], dt, "cuda") for n in NAMES}
    s0 = None if inp["s0"] is None else torch.from_numpy(inp["s0"]).cuda()
    dsf = None if d_sf is None else torch.from_numpy(d_sf).cuda()
    g = wkv7.gdn_bwd(*(dev[n] for n in NAMES), synth.to_torch(d_o, dt, "cuda"), initial_state=s0,
                     d_final_state=dsf, workspace=workspace)
    torch.cuda.synchronize()
    return {n: hz.to_np(x) for n, x in g.items()}


def oracle_bwd(inp, d_o, d_sf):
    return oracle.gdn_bwd(*(inp[n] for n in NAMES), d_o, inp["s0"], d_sf)


def check_all(dtype, g, ref, what):
    for n in NAMES:
        check_grad(dtype, g[n], ref[n], f"{what} d{n}")
    check_grad("f32", g["s0"], ref["s0"], f"{what} ds0")


@pytest.mark.parametrize("dtype,D,B,T,H,init,n_state,dsf", [
    ("f32", 64, 2, 50, 2, True, None, True),
    ("f32", 128, 1, 40, 2, True, None, True),
    ("f32", 64, 3, 33, 1, True, 1, True),         # one shared initial state
    ("f32", 64, 1, 16, 1, False, None, False),
    ("bf16", 64, 2, 200, 2, True, None, True),
    ("bf16", 128, 2, 130, 1, True, 1, True),
    ("bf16", 64, 3, 77, 3, False, None, False),
    ("bf16", 128, 1, 61, 2, False, None, True),
])
def test_gdn_bwd_parity(dtype, D, B, T, H, init, n_state, dsf):
    inp, d_o, d_sf = make_case(B, T, H, D, dtype, seed=7000 + T + D, init=init, n_state=n_state, dsf=dsf)
    g = run_gpu(inp, d_o, d_sf)
    check_all(dtype, g, oracle_bwd(inp, d_o, d_sf), f"gdn bwd {dtype} D{D} T{T}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 33])
def test_gdn_bwd_short_and_ragged(D, T):
    inp, d_o, d_sf = make_case(2, T, 1, D, "f32", seed=7200 + T, n_state=1)
    g = run_gpu(inp, d_o, d_sf)
    check_all("f32", g, oracle_bwd(inp, d_o, d_sf), f"gdn bwd ragged D{D} T{T}")


def test_gdn_bwd_strong_gates():
    """Gates of -20 on whole chunks (the exact token-by-token path of the
    WKV7 backward), a token with beta = 1 and g = 0 (a pure replacement of
    the kn direction) and one with beta = 0 (no write)."""
    B, T, H, D = 2, 80, 1, 64
    inp, d_o, d_sf = make_case(B, T, H, D, "f32", seed=7300)
    inp["g"][0, 16:32] = -20.0
    inp["g"][1, 40] = 0.0
    inp["beta"][1, 40] = 1.0
    inp["beta"][0, 50] = 0.0
    g = run_gpu(inp, d_o, d_sf)
    check_all("f32", g, oracle_bwd(inp, d_o, d_sf), "gdn bwd strong gates")


def test_gdn_bwd_empty_sequence_shared_state():
    inp, d_o, d_sf = make_case(3, 0, 2, 64, "f32", seed=7400, n_state=1)
    g = run_gpu(inp, d_o, d_sf)
    np.testing.assert_allclose(g["s0"][0], d_sf.astype(np.float64).sum(axis=0), rtol=1e-6, atol=1e-6)
    assert g["q"].shape == (3, 0, 2, 64) and g["g"].shape == (3, 0, 2)


def test_gdn_bwd_full_size_sampled():
    """The Gated DeltaNet benchmark shape (B8 T4096 H64 d64, bf16), checked
    on sampled (sequence, head) pairs that the oracle recomputes alone."""
    B, T, H, D = 8, 4096, 64, 64
    inp, d_o, d_sf = make_case(B, T, H, D, "bf16", seed=7500, init=False, dsf=False)
    g = run_gpu(inp, d_o, d_sf)
    rng = np.random.default_rng(7501)
    for bb, h in zip(rng.integers(0, B, 2), rng.integers(0, H, 2)):
        sl = {n: inp[n][bb:bb + 1, :, h:h + 1] for n in NAMES}
        ref = oracle.gdn_bwd(*(sl[n] for n in NAMES), d_o[bb:bb + 1, :, h:h + 1])
        for n in ("q", "k", "v"):
            check_grad("bf16", g[n][bb, :, h], ref[n][0, :, 0], f"gdn bwd full b{bb} h{h} d{n}")
        for n in ("g", "beta"):
            check_grad("bf16", g[n][bb, :, h], ref[n][0, :, 0], f"gdn bwd full b{bb} h{h} d{n}")
        check_grad("f32", g["s0"][bb, h], ref["s0"][0, 0], f"gdn bwd full b{bb} h{h} ds0")


def test_gdn_bwd_reused_workspace_and_deterministic():
    """Two calls through one workspace (the second on a smaller problem)
    each match their own fresh-workspace result bit for bit."""
    big = make_case(2, 100, 4, 64, "bf16", seed=7600, n_state=1)
    small = make_case(1, 40, 2, 64, "bf16", seed=7601)
    ws = torch.empty(wkv7.gdn_bwd_workspace_bytes(2, 100, 4, 64, 64), dtype=torch.uint8, device="cuda")
    g1 = run_gpu(*big, workspace=ws)
    g2 = run_gpu(*small, workspace=ws)
    for case, got in ((big, g1), (small, g2)):
        fresh = run_gpu(*case)
        for n in got:
            np.testing.assert_array_equal(got[n], fresh[n], err_msg=n)


@pytest.mark.parametrize("dtype,D,mapped", [("bf16", 64, True), ("f32", 64, False), ("bf16", 128, False)])
def test_gdn_bwd_varlen_parity(dtype, D, mapped):
    """Packed sequences (wkv7_gdn_bwd_varlen) against the oracle run on each
    sequence alone, starting from its pool row (a state_map entry outside
    the pool: zero state; no map and one pool row: that row for every
    sequence)."""
    lengths, H = [0, 30, 17, 64], 2
    TT, N = sum(lengths), len(lengths)
    gi = synth.make_gdn(1, TT, H, D, seed=7700 + D, dtype=dtype)
    rng = np.random.default_rng(7701)
    n_state = 3 if mapped else 1
    pool = (rng.standard_normal((n_state, H, D, D)) * 0.1).astype(np.float32)
    smap = np.array([1, 2, -1, 0], np.int32) if mapped else None
    d_o = synth.round_to(rng.standard_normal((TT, H, D)).astype(np.float32), dtype)
    d_sf = (rng.standard_normal((N, H, D, D)) * 0.5).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = {n: synth.to_torch(gi[n][0], dtype, "cuda") for n in NAMES}
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    g = wkv7.gdn_bwd_varlen(*(dev[n] for n in NAMES), t(cu), synth.to_torch(d_o, dtype, "cuda"),
                            initial_state=t(pool), state_map=t(smap), d_final_state=t(d_sf))
    torch.cuda.synchronize()
    g = {n: hz.to_np(x) for n, x in g.items()}
    for n in range(N):
        tb, te = int(cu[n]), int(cu[n + 1])
        row = (int(smap[n]) if mapped else 0)
        s0 = pool[row][None] if 0 <= row < n_state else None
        if te == tb:
            np.testing.assert_array_equal(g["s0"][n], d_sf[n])
            continue
        sl = {k: gi[k][:, tb:te] for k in NAMES}
        ref = oracle.gdn_bwd(*(sl[k] for k in NAMES), d_o[tb:te][None], s0, d_sf[n][None])
        for k in NAMES:
            check_grad(dtype, g[k][tb:te], ref[k][0], f"gdn bwd varlen {dtype} D{D} seq{n} d{k}")
        check_grad("f32", g["s0"][n], ref["s0"][0], f"gdn bwd varlen {dtype} D{D} seq{n} ds0")


@pytest.mark.parametrize("N", [128, 129])
def test_gdn_bwd_varlen_many_sequences_with_equal_lengths(N):
    """Many packed sequences with repeated lengths (ties in the recurrences'
    longest-first order), at and just past the largest count that order
    covers: every sequence's gradients against the oracle.  A one-token
    sequence from a zero state has dg = 0 identically (the gate only scales
    a zero state); the documented floor, the sequence's gradient RMS,
    applies to such tensors alone."""
    rng = np.random.default_rng(7800 + N)
    lengths = rng.choice([0, 1, 17, 400, 517, 600, 700], size=N).tolist()
    assert N > 128 or sum(lengths) >= 256 * N   # the longest-first order applies
    TT, H, D = sum(lengths), 2, 64
    gi = synth.make_gdn(1, TT, H, D, seed=7801 + N, dtype="bf16")
    pool = (rng.standard_normal((3, H, D, D)) * 0.1).astype(np.float32)
    smap = rng.integers(-1, 4, size=N).astype(np.int32)
    d_o = synth.round_to(rng.standard_normal((TT, H, D)).astype(np.float32), "bf16")
    d_sf = (rng.standard_normal((N, H, D, D)) * 0.5).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = {n: synth.to_torch(gi[n][0], "bf16", "cuda") for n in NAMES}
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    g = wkv7.gdn_bwd_varlen(*(dev[n] for n in NAMES), t(cu), synth.to_torch(d_o, "bf16", "cuda"),
                            initial_state=t(pool), state_map=t(smap), d_final_state=t(d_sf))
    torch.cuda.synchronize()
    g = {n: hz.to_np(x) for n, x in g.items()}
    for n in range(N):
        tb, te = int(cu[n]), int(cu[n + 1])
        row = int(smap[n])
        s0 = pool[row][None] if 0 <= row < 3 else None
        if te == tb:
            np.testing.assert_array_equal(g["s0"][n], d_sf[n])
            continue
        sl = {k: gi[k][:, tb:te] for k in NAMES}
        ref = oracle.gdn_bwd(*(sl[k] for k in NAMES), d_o[tb:te][None], s0, d_sf[n][None])
        fl = float(np.sqrt(np.mean(np.concatenate([ref[k].ravel() for k in NAMES]) ** 2)))
        for k in NAMES:
            check_grad("bf16", g[k][tb:te], ref[k][0], f"gdn bwd varlen N={N} seq{n} d{k}", floor=fl)
        check_grad("f32", g["s0"][n], ref["s0"][0], f"gdn bwd varlen N={N} seq{n} ds0")

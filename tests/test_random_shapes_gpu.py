"""Seeded random shapes through every sequence-level entry point, against
the fp64 oracle: odd B, T and H, both head sizes, both I/O types, with and
without initial state and mask, and packed batches of random lengths
(including empty ones).  The tolerances are those of the dedicated tests
(tests/harness.py for outputs, tests/test_bwd_gpu.py for gradients)."""
import numpy as np
import pytest

import harness as hz
import oracle
from rwkv_linear_attention_amd import synth, wkv7
from harness import check_grad


def grad_scale(ref, names):
    """RMS over all input gradients of one call: the scale floor for a
    gradient tensor that vanishes identically (see check_grad)."""
    return float(np.sqrt(np.mean(np.concatenate([np.ravel(ref[n]) for n in names]) ** 2)))

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("r", "w", "k", "v", "a", "b")
GNAMES = ("q", "k", "v", "g", "beta")


def draw(seed):
    rng = np.random.default_rng(seed)
    return dict(B=int(rng.integers(1, 4)), T=int(rng.integers(1, 90)), H=int(rng.integers(1, 4)),
                D=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
                init=bool(rng.integers(0, 2)), mask=str(rng.choice(["none", "bernoulli", "trailing"])))


@pytest.mark.parametrize("seed", range(8))
def test_random_fwd_and_bwd(seed):
    c = draw(10_000 + seed)
    inp = synth.make(1, B=c["B"], T=c["T"], H=c["H"], K=c["D"], seed=10_100 + seed, init=c["init"], mask=c["mask"])
    dt = c["dtype"]
    for n in NAMES:
        inp[n] = synth.round_to(inp[n], dt)
    dev = {n: synth.to_torch(inp[n], dt, "cuda") for n in NAMES}
    s0 = None if inp["s0"] is None else torch.from_numpy(inp["s0"]).cuda()
    mask = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).cuda()
    o, sf = wkv7.fwd(*(dev[n] for n in NAMES), initial_state=s0, mask=mask)
    rng = np.random.default_rng(10_200 + seed)
    d_o = synth.round_to(rng.standard_normal(inp["v"].shape).astype(np.float32), dt)
    g = wkv7.bwd(*(dev[n] for n in NAMES), synth.to_torch(d_o, dt, "cuda"), initial_state=s0, mask=mask)
    torch.cuda.synchronize()
    what = f"random {seed} {c}"
    o_ref, s_ref = oracle.fwd(*(inp[n] for n in NAMES), inp["s0"], inp["mask"])
    hz.check(dt, hz.to_np(o), o_ref, hz.to_np(sf), s_ref, what=what + " fwd")
    ref = oracle.bwd(*(inp[n] for n in NAMES), d_o, inp["s0"], inp["mask"])
    fl = grad_scale(ref, NAMES)
    for n in NAMES:
        check_grad(dt, hz.to_np(g[n]), ref[n], f"{what} d{n}", floor=fl)
    check_grad("f32", hz.to_np(g["s0"]), ref["s0"], f"{what} ds0")


@pytest.mark.parametrize("seed", range(6))
def test_random_gdn_fwd_and_bwd(seed):
    c = draw(11_000 + seed)
    n_state = None if not c["init"] else (1 if seed % 2 else c["B"])
    gi = synth.make_gdn(c["B"], c["T"], c["H"], c["D"], seed=11_100 + seed, dtype=c["dtype"], init=c["init"],
                        n_state=n_state)
    dt = c["dtype"]
    dev = {n: synth.to_torch(gi[n], dt, "cuda") for n in GNAMES}
    s0 = None if gi["s0"] is None else torch.from_numpy(gi["s0"]).cuda()
    o, sf = wkv7.gdn_fwd(*(dev[n] for n in GNAMES), initial_state=s0)
    rng = np.random.default_rng(11_200 + seed)
    d_o = synth.round_to(rng.standard_normal(gi["v"].shape).astype(np.float32), dt)
    g = wkv7.gdn_bwd(*(dev[n] for n in GNAMES), synth.to_torch(d_o, dt, "cuda"), initial_state=s0)
    torch.cuda.synchronize()
    what = f"random gdn {seed} {c}"
    o_ref, s_ref = oracle.gdn_fwd(*(gi[n] for n in GNAMES), gi["s0"])
    hz.check(dt, hz.to_np(o), o_ref, hz.to_np(sf), s_ref, what=what + " fwd")
    ref = oracle.gdn_bwd(*(gi[n] for n in GNAMES), d_o, gi["s0"])
    fl = grad_scale(ref, GNAMES)
    for n in GNAMES:
        check_grad(dt, hz.to_np(g[n]), ref[n], f"{what} d{n}", floor=fl)
    check_grad("f32", hz.to_np(g["s0"]), ref["s0"], f"{what} ds0")


@pytest.mark.parametrize("seed", range(4))
def test_random_packed_fwd_and_bwd(seed):
    rng = np.random.default_rng(12_000 + seed)
    N, H, D = int(rng.integers(1, 6)), int(rng.integers(1, 3)), int(rng.choice([64, 128]))
    lengths = [int(x) for x in rng.integers(0, 70, size=N)]
    TT = sum(lengths)
    dt = "bf16"
    inp = synth.make(1, B=1, T=max(TT, 1), H=H, K=D, seed=12_100 + seed, mask="bernoulli")
    x = {n: synth.round_to(inp[n][0, :TT], dt) for n in NAMES}
    mask = inp["mask"][0, :TT]
    n_state = int(rng.integers(1, 4))
    pool = (rng.standard_normal((n_state, H, D, D)) * 0.1).astype(np.float32)
    smap = rng.integers(-1, n_state + 1, size=N).astype(np.int32)     # includes out-of-range rows
    d_o = synth.round_to(rng.standard_normal((TT, H, D)).astype(np.float32), dt)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dev = {n: synth.to_torch(x[n], dt, "cuda") for n in NAMES}
    o, sf = wkv7.fwd_varlen(*(dev[n] for n in NAMES), t(cu), initial_state=t(pool), state_map=t(smap), mask=t(mask))
    g = wkv7.bwd_varlen(*(dev[n] for n in NAMES), t(cu), synth.to_torch(d_o, dt, "cuda"), initial_state=t(pool),
                        state_map=t(smap), mask=t(mask))
    torch.cuda.synchronize()
    o, sf = hz.to_np(o), hz.to_np(sf)
    g = {n: hz.to_np(v) for n, v in g.items()}
    for n in range(N):
        tb, te = int(cu[n]), int(cu[n + 1])
        row = int(smap[n])
        s0 = pool[row][None] if 0 <= row < n_state else None
        what = f"random packed {seed} seq{n} (len {te - tb}, D{D})"
        if te == tb:
            np.testing.assert_array_equal(sf[n], np.zeros_like(sf[n]) if s0 is None else s0[0])
            np.testing.assert_array_equal(g["s0"][n], 0.0)
            continue
        sl = {k: x[k][tb:te][None] for k in NAMES}
        o_ref, s_ref = oracle.fwd(*(sl[k] for k in NAMES), s0, mask[tb:te][None])
        hz.check(dt, o[tb:te], o_ref[0], sf[n], s_ref[0], what=what + " fwd")
        ref = oracle.bwd(*(sl[k] for k in NAMES), d_o[tb:te][None], s0, mask[tb:te][None])
        fl = grad_scale(ref, NAMES)
        for k in NAMES:
            check_grad(dt, g[k][tb:te], ref[k][0], f"{what} d{k}", floor=fl)
        check_grad("f32", g["s0"][n], ref["s0"][0], f"{what} ds0")

"""GPU checks of the interface details around the kernels:

- one initial state shared by every sequence ([1,H,K,V], the form in the
  rwkv-ops README argument tables) through wkv7_fwd, wkv7_bwd and the packed
  entries without a state_map;
- the packed entries under AUTO take the chunked kernel whatever the
  lengths (a skewed batch of many one-token sequences and one long one);
- tokens outside every packed sequence read as zero in the outputs and the
  gradients of the Python wrappers;
- a hand-off wait of the chunked kernel that gives up poisons its results
  with NaN (forced from the host with the wait-limit hook; every kernel
  still exits normally).

Expected values come from the fp64 oracle: a shared state is the same
initial state given to every sequence, and its gradient is the sum of the
per-sequence gradients.
"""
import numpy as np
import pytest

import harness as hz
import oracle
from harness import check_grad
from rwkv_linear_attention_amd import synth, wkv7

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("r", "w", "k", "v", "a", "b")
REC, CHK = wkv7.ALGO_RECURRENT, wkv7.ALGO_CHUNKED


def _dev(inp, dt):
    return {n: synth.to_torch(inp[n], dt, "cuda") for n in NAMES}


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("algo", [REC, CHK])
def test_fwd_shared_initial_state(D, algo):
    B, T, H = 3, 70, 2
    inp = synth.make(1, B=B, T=T, H=H, K=D, seed=700 + D, init=False, mask="bernoulli")
    s1 = (np.random.default_rng(701).standard_normal((1, H, D, D)) * 0.1).astype(np.float32)
    dev = _dev(inp, "bf16")
    s1_t = torch.from_numpy(s1).cuda()
    mask = torch.from_numpy(inp["mask"]).cuda()
    o, sf = wkv7.fwd(*(dev[n] for n in NAMES), initial_state=s1_t, mask=mask, algo=algo)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd(*(inp[n] for n in NAMES), np.repeat(s1, B, axis=0), inp["mask"])
    hz.check("bf16", hz.to_np(o), o_ref, hz.to_np(sf), s_ref, f"shared state fwd D{D} algo {algo}")
    # the same rows given explicitly give bit-identical results
    o2, sf2 = wkv7.fwd(*(dev[n] for n in NAMES), initial_state=s1_t.expand(B, -1, -1, -1).contiguous(),
                       mask=mask, algo=algo)
    assert torch.equal(o, o2) and torch.equal(sf, sf2)
    # T = 0 copies the shared state into every final row
    empty = {n: dev[n][:, :0].contiguous() for n in NAMES}
    _, sf0 = wkv7.fwd(*(empty[n] for n in NAMES), initial_state=s1_t)
    torch.cuda.synchronize()
    assert all(torch.equal(sf0[i], s1_t[0]) for i in range(B))


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 128)])
def test_bwd_shared_initial_state(dtype, D):
    B, T, H = 3, 50, 2
    inp = synth.make(1, B=B, T=T, H=H, K=D, seed=710 + D, init=False, mask="trailing")
    for n in NAMES:
        inp[n] = synth.round_to(inp[n], dtype)
    rng = np.random.default_rng(711)
    s1 = (rng.standard_normal((1, H, D, D)) * 0.1).astype(np.float32)
    d_o = synth.round_to(rng.standard_normal((B, T, H, D)).astype(np.float32), dtype)
    d_sf = (rng.standard_normal((B, H, D, D)) * 0.5).astype(np.float32)
    dev = _dev(inp, dtype)
    g = wkv7.bwd(*(dev[n] for n in NAMES), synth.to_torch(d_o, dtype, "cuda"),
                 initial_state=torch.from_numpy(s1).cuda(), mask=torch.from_numpy(inp["mask"]).cuda(),
                 d_final_state=torch.from_numpy(d_sf).cuda())
    torch.cuda.synchronize()
    assert tuple(g["s0"].shape) == (1, H, D, D)
    ref = oracle.bwd(*(inp[n] for n in NAMES), d_o, np.repeat(s1, B, axis=0), inp["mask"], d_sf)
    for n in NAMES:
        check_grad(dtype, hz.to_np(g[n]), ref[n], f"shared state bwd D{D} d{n}")
    check_grad("f32", hz.to_np(g["s0"]), ref["s0"].sum(axis=0, keepdims=True), f"shared state bwd D{D} ds0")


def test_bwd_shared_initial_state_empty():
    """T = 0: the shared state's gradient is the sum of the final-state gradients."""
    B, H, D = 3, 2, 64
    z = torch.zeros((B, 0, H, D), dtype=torch.bfloat16, device="cuda")
    s1 = torch.randn((1, H, D, D), device="cuda")
    d_sf = torch.randn((B, H, D, D), device="cuda")
    g = wkv7.bwd(z, z, z, z, z, z, z, initial_state=s1, d_final_state=d_sf)
    torch.cuda.synchronize()
    exp = d_sf[0] + d_sf[1] + d_sf[2]
    assert torch.allclose(g["s0"][0], exp, rtol=0, atol=1e-6)


@pytest.mark.parametrize("algo", [wkv7.ALGO_AUTO, REC])
def test_packed_one_row_pool_without_map(algo):
    """A one-row pool without state_map is shared by every packed sequence,
    in the forward and the backward."""
    H, D = 2, 64
    lengths = [30, 1, 47]
    TT = sum(lengths)
    inp = synth.make(1, B=1, T=TT, H=H, K=D, seed=720, init=False, mask="bernoulli")
    x = {n: inp[n][0] for n in NAMES}
    m = inp["mask"][0]
    rng = np.random.default_rng(721)
    s1 = (rng.standard_normal((1, H, D, D)) * 0.1).astype(np.float32)
    d_o = synth.round_to(rng.standard_normal((TT, H, D)).astype(np.float32), "bf16")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = {n: synth.to_torch(x[n], "bf16", "cuda") for n in NAMES}
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o, sf = wkv7.fwd_varlen(*(dev[n] for n in NAMES), t(cu), initial_state=t(s1), mask=t(m), algo=algo)
    g = wkv7.bwd_varlen(*(dev[n] for n in NAMES), t(cu), synth.to_torch(d_o, "bf16", "cuda"),
                        initial_state=t(s1), mask=t(m))
    torch.cuda.synchronize()
    o, sf = hz.to_np(o), hz.to_np(sf)
    g = {n: hz.to_np(v) for n, v in g.items()}
    for n in range(len(lengths)):
        tb, te = int(cu[n]), int(cu[n + 1])
        sl = {k: x[k][tb:te][None] for k in NAMES}
        o_ref, s_ref = oracle.fwd(*(sl[k] for k in NAMES), s1, m[tb:te][None])
        hz.check("bf16", o[tb:te], o_ref[0], sf[n], s_ref[0], f"one-row pool seq {n}")
        ref = oracle.bwd(*(sl[k] for k in NAMES), d_o[tb:te][None], s1, m[tb:te][None])
        for k in NAMES:
            check_grad("bf16", g[k][tb:te], ref[k][0], f"one-row pool seq {n} d{k}")
        check_grad("f32", g["s0"][n], ref["s0"][0], f"one-row pool seq {n} ds0")


@pytest.mark.parametrize("D", [64, 128])
def test_packed_auto_takes_chunked_on_skewed_batch(D):
    """299 one-token sequences and one of 4096 tokens: a mean length below
    16, which a mean-length rule would send to the recurrent kernel.  AUTO
    must give exactly the chunked kernel's results (the recurrent kernel
    rounds differently), and the long sequence must match the oracle."""
    H = 2
    lengths = [1] * 299 + [4096]
    TT = sum(lengths)
    inp = synth.make(1, B=1, T=TT, H=H, K=D, seed=730 + D, init=False, mask="none")
    x = {n: inp[n][0] for n in NAMES}
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).cuda()
    dev = {n: synth.to_torch(x[n], "bf16", "cuda") for n in NAMES}
    o_auto, s_auto = wkv7.fwd_varlen(*(dev[n] for n in NAMES), cu, algo=wkv7.ALGO_AUTO)
    o_chk, s_chk = wkv7.fwd_varlen(*(dev[n] for n in NAMES), cu, algo=CHK)
    o_rec, _ = wkv7.fwd_varlen(*(dev[n] for n in NAMES), cu, algo=REC)
    torch.cuda.synchronize()
    assert torch.equal(o_auto, o_chk) and torch.equal(s_auto, s_chk)
    assert not torch.equal(o_auto, o_rec)
    tb = 299
    sl = {k: x[k][tb:][None] for k in NAMES}
    o_ref, s_ref = oracle.fwd(*(sl[k] for k in NAMES))
    hz.check("bf16", hz.to_np(o_auto[tb:]), o_ref[0], hz.to_np(s_auto[299]), s_ref[0], f"skewed long seq D{D}")


def test_packed_uncovered_tokens_are_zero():
    """cu_seqlens starting after token 0 and ending before the last token
    (leading and trailing padding in a packed buffer): the wrappers' output
    and input gradients there are zero, whatever the padding holds, and the
    covered tokens still match the oracle."""
    H, D, TT = 2, 64, 120
    inp = synth.make(1, B=1, T=TT, H=H, K=D, seed=740, init=False, mask="none")
    x = {n: inp[n][0] for n in NAMES}
    rng = np.random.default_rng(741)
    d_o = synth.round_to(rng.standard_normal((TT, H, D)).astype(np.float32), "bf16")
    cu_np = np.array([10, 40, 90], np.int32)          # sequences [10, 40) and [40, 90)
    dev = {n: synth.to_torch(x[n], "bf16", "cuda") for n in NAMES}
    for n in NAMES:                                    # padding the operator must never read
        dev[n][:10] = float("nan")
        dev[n][90:] = float("inf")
    cu = torch.from_numpy(cu_np).cuda()
    d_o_t = synth.to_torch(d_o, "bf16", "cuda")
    for algo in (CHK, REC):
        o, sf = wkv7.fwd_varlen(*(dev[n] for n in NAMES), cu, algo=algo)
        g = wkv7.bwd_varlen(*(dev[n] for n in NAMES), cu, d_o_t)
        torch.cuda.synchronize()
        o_np = hz.to_np(o)
        assert np.all(o_np[:10] == 0.0) and np.all(o_np[90:] == 0.0), f"algo {algo}: padding output"
        for n in NAMES:
            gn = hz.to_np(g[n])
            assert np.all(gn[:10] == 0.0) and np.all(gn[90:] == 0.0), f"d{n} at padding"
        for i in range(2):
            tb, te = int(cu_np[i]), int(cu_np[i + 1])
            sl = {k: x[k][tb:te][None] for k in NAMES}
            o_ref, s_ref = oracle.fwd(*(sl[k] for k in NAMES))
            hz.check("bf16", o_np[tb:te], o_ref[0], hz.to_np(sf[i]), s_ref[0], f"padded seq {i} algo {algo}")
            ref = oracle.bwd(*(sl[k] for k in NAMES), d_o[tb:te][None])
            for k in NAMES:
                check_grad("bf16", hz.to_np(g[k])[tb:te], ref[k][0], f"padded seq {i} d{k}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gdn", [False, True])
def test_handoff_give_up_poisons_results(D, gdn):
    """With the wait limit at 0 every hand-off wait of the chunked kernel
    gives up at once: every output and final state must then be NaN, and the
    kernel must still finish.  After the default is restored the same call
    matches the oracle again."""
    B, T, H = 2, 100, 2
    prev = wkv7.set_wait_limit(0)
    try:
        if gdn:
            gi = synth.make_gdn(B, T, H, D, seed=750 + D, init=True)
            dv = {n: synth.to_torch(gi[n], "bf16", "cuda") for n in ("q", "k", "v", "g", "beta")}
            call = lambda: wkv7.gdn_fwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"],
                                        initial_state=torch.from_numpy(gi["s0"]).cuda(), algo=CHK)
        else:
            inp = synth.make(1, B=B, T=T, H=H, K=D, seed=750 + D, init=True, mask="bernoulli")
            dev = hz.to_dev(inp)
            call = lambda: hz.gpu_fwd(dev, algo=CHK)
        o, sf = call()
        torch.cuda.synchronize()
        assert torch.isnan(o.float()).all(), "outputs after a give-up must be NaN"
        assert torch.isnan(sf).all(), "final states after a give-up must be NaN"
    finally:
        wkv7.set_wait_limit(prev)
    o, sf = call()
    torch.cuda.synchronize()
    if gdn:
        o_ref, s_ref = oracle.gdn_fwd(gi["q"], gi["k"], gi["v"], gi["g"], gi["beta"], gi["s0"])
    else:
        o_ref, s_ref = hz.oracle_fwd(inp)
    hz.check("bf16", hz.to_np(o), o_ref, hz.to_np(sf), s_ref, f"after give-up test D{D} gdn={gdn}")

"""GPU parity of wkv7_gdn_fwd (Gated DeltaNet on the generalized-delta-rule
kernels) against the fp64 oracle's textbook gated delta rule.

Inputs follow the argument table of the rwkv-ops README, section
"gdn_recurrent 使用方法" (q, k raw and normalised inside, log-space gate g,
strength beta in (0, 1), initial state with B rows or one shared row).
Tolerances are the ones of the WKV7 forward (tests/harness.py).
"""
import numpy as np
import pytest

import harness as hz
import oracle
from rwkv_linear_attention_amd import synth, wkv7

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REC, CHK = wkv7.ALGO_RECURRENT, wkv7.ALGO_CHUNKED
NAMES = ("q", "k", "v", "g", "beta")


def to_dev(inp):
    dt = inp["dtype"]
    dev = {n: synth.to_torch(inp[n], dt, "cuda") for n in NAMES}
    dev["s0"] = None if inp["s0"] is None else torch.from_numpy(inp["s0"]).cuda()
    return dev


def run(dev, algo, **kw):
    o, sf = wkv7.gdn_fwd(*(dev[n] for n in NAMES), initial_state=dev["s0"], algo=algo, **kw)
    torch.cuda.synchronize()
    return o, sf


def ref(inp):
    return oracle.gdn_fwd(*(inp[n] for n in NAMES), inp["s0"])


CASES = [
    # (dtype, D, algo, B, T, H, init, n_state)
    ("bf16", 64, CHK, 2, 200, 2, True, None),
    ("bf16", 128, CHK, 2, 200, 2, True, None),
    ("bf16", 64, CHK, 3, 77, 2, True, 1),
    ("bf16", 128, CHK, 3, 77, 1, True, 1),
    ("bf16", 64, CHK, 2, 64, 3, False, None),
    ("bf16", 64, REC, 2, 200, 2, True, None),
    ("bf16", 128, REC, 2, 90, 2, True, 1),
    ("f32", 64, REC, 2, 130, 2, True, None),
    ("f32", 128, REC, 2, 70, 1, True, 1),
    ("f32", 64, REC, 1, 33, 2, False, None),
]


@pytest.mark.parametrize("dtype,D,algo,B,T,H,init,n_state", CASES)
def test_gdn_parity(dtype, D, algo, B, T, H, init, n_state):
    inp = synth.make_gdn(B, T, H, D, seed=4100 + D + T, dtype=dtype, init=init, n_state=n_state)
    o, sf = run(to_dev(inp), algo)
    o_ref, s_ref = ref(inp)
    hz.check(dtype, hz.to_np(o), o_ref, hz.to_np(sf), s_ref, what=f"gdn {dtype} D{D} algo{algo} T{T}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 31, 33])
def test_gdn_chunked_short_and_ragged(D, T):
    inp = synth.make_gdn(2, T, 2, D, seed=4300 + T, init=True)
    o, sf = run(to_dev(inp), CHK)
    o_ref, s_ref = ref(inp)
    hz.check("bf16", hz.to_np(o), o_ref, hz.to_np(sf), s_ref, what=f"gdn ragged D{D} T{T}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("algo", [REC, CHK])
def test_gdn_extreme_gates(D, algo):
    """Gates of -20 drive the decay of whole chunks below any fp32 range
    (the chunked kernel then takes its exact per-token path); gates of 0 keep
    the state undecayed.  Both must still match the recurrence."""
    B, T, H = 2, 96, 2
    inp = synth.make_gdn(B, T, H, D, seed=4400 + D, init=True)
    g = inp["g"].copy()
    g[0, 16:48] = -20.0            # two whole chunks of sequence 0 forget everything
    g[1, 40:44] = -20.0            # a few tokens inside one chunk of sequence 1
    g[:, 64:80] = 0.0              # one chunk without decay
    inp["g"] = synth.round_to(g, "bf16")
    o, sf = run(to_dev(inp), algo)
    o_ref, s_ref = ref(inp)
    hz.check("bf16", hz.to_np(o), o_ref, hz.to_np(sf), s_ref, what=f"gdn extreme D{D} algo{algo}")


def test_gdn_state_in_place_and_empty():
    inp = synth.make_gdn(2, 48, 2, 64, seed=4500, init=True)
    dev = to_dev(inp)
    s = dev["s0"].clone()
    o, sf = wkv7.gdn_fwd(*(dev[n] for n in NAMES), initial_state=s, final_state=s, algo=CHK)
    torch.cuda.synchronize()
    assert sf.data_ptr() == s.data_ptr()
    o_ref, s_ref = ref(inp)
    hz.check("bf16", hz.to_np(o), o_ref, hz.to_np(s), s_ref, what="gdn in-place")
    # T == 0 with a shared state: every sequence's final state is that state
    empty = synth.make_gdn(3, 0, 2, 64, seed=4501, init=True, n_state=1)
    de = to_dev(empty)
    o0, sf0 = wkv7.gdn_fwd(*(de[n] for n in NAMES), initial_state=de["s0"])
    torch.cuda.synchronize()
    assert o0.shape == (3, 0, 2, 64)
    np.testing.assert_array_equal(sf0.cpu().numpy(), np.broadcast_to(empty["s0"], (3, 2, 64, 64)))


def test_gdn_rejects_aliased_shared_state():
    """A shared initial state that is also the final-state buffer would be
    overwritten while other sequences still read it: the library refuses."""
    inp = synth.make_gdn(2, 16, 1, 64, seed=4502, init=True, n_state=1)
    dev = to_dev(inp)
    buf = torch.zeros((2, 1, 64, 64), dtype=torch.float32, device="cuda")
    buf[:1].copy_(dev["s0"])
    with pytest.raises(wkv7.WKV7Error):
        wkv7.gdn_fwd(*(dev[n] for n in NAMES), initial_state=buf[:1], final_state=buf)


@pytest.mark.parametrize("D,B,H", [(64, 8, 64), (128, 16, 32)])
def test_gdn_full_size_sampled(D, B, H):
    """Full-size launch (T = 4096, as timed by the benchmark) checked on
    sampled (sequence, head) pairs, each recomputed by the oracle alone."""
    T = 4096
    inp = synth.make_gdn(B, T, H, D, seed=4600 + D, init=False)
    o, sf = run(to_dev(inp), CHK)
    o, sf = hz.to_np(o), hz.to_np(sf)
    rng = np.random.default_rng(4601)
    for bb, h in zip(rng.integers(0, B, 3), rng.integers(0, H, 3)):
        sl = {n: inp[n][bb:bb + 1, :, h:h + 1] for n in NAMES}
        o_ref, s_ref = oracle.gdn_fwd(*(sl[n] for n in NAMES), None)
        hz.check("bf16", o[bb, :, h], o_ref[0, :, 0], sf[bb, h], s_ref[0, 0], what=f"gdn full D{D} b{bb} h{h}")


@pytest.mark.parametrize("dtype,D,state", [("bf16", 64, "own"), ("bf16", 128, "shared"), ("f32", 64, "none"),
                                           ("f32", 128, "own"), ("bf16", 64, "shared")])
def test_gdn_step_matches_oracle(dtype, D, state):
    """Single-token decode (the T = 1 case of the forward): output and next
    state against the oracle's gated delta rule."""
    B, H = 5, 3
    inp = synth.make_gdn(B, 1, H, D, seed=4700 + D, dtype=dtype, init=state != "none",
                         n_state=1 if state == "shared" else None)
    dev = to_dev(inp)
    one = {n: dev[n][:, 0].contiguous() for n in NAMES}
    s_in = dev["s0"]
    o, s_next = wkv7.gdn_step(*(one[n] for n in NAMES), state=s_in)
    torch.cuda.synchronize()
    if state == "own":
        assert s_next.data_ptr() == s_in.data_ptr()      # B rows: updated in place
    o_ref, s_ref = ref(inp)
    hz.check(dtype, hz.to_np(o), o_ref[:, 0], hz.to_np(s_next), s_ref, what=f"gdn step {dtype} D{D} {state}")


@pytest.mark.parametrize("D", [64, 128])
def test_gdn_steps_equal_forward(D):
    """Twelve consecutive in-place decode steps reproduce the oracle's
    forward over the same twelve tokens."""
    B, T, H = 3, 12, 2
    inp = synth.make_gdn(B, T, H, D, seed=4800 + D, init=True)
    dev = to_dev(inp)
    state = dev["s0"].clone()
    outs = []
    for t in range(T):
        o, state = wkv7.gdn_step(*(dev[n][:, t].contiguous() for n in NAMES), state=state)
        outs.append(hz.to_np(o))
    torch.cuda.synchronize()
    o_ref, s_ref = ref(inp)
    hz.check("bf16", np.stack(outs, axis=1), o_ref, hz.to_np(state), s_ref, what=f"gdn steps D{D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("algo", [REC, CHK])
@pytest.mark.parametrize("pool", ["map", "shared", "rows"])
def test_gdn_varlen(D, algo, pool):
    """Packed sequences (mixed lengths, one empty) are independent runs of the
    Gated DeltaNet forward, each from its pool row."""
    lengths = [37, 0, 16, 101, 5]
    N, TT, H = len(lengths), sum(lengths), 2
    inp = synth.make_gdn(1, TT, H, D, seed=4900 + D, init=False)
    rng = np.random.default_rng(4901)
    n_pool = {"map": 3, "shared": 1, "rows": N}[pool]
    poolv = (rng.standard_normal((n_pool, H, D, D)) * 0.1).astype(np.float32)
    smap = np.array([2, 0, 7, 1, 2], np.int32) if pool == "map" else None     # 7: out of range -> zeros
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = {n: synth.to_torch(inp[n][0], "bf16", "cuda") for n in NAMES}
    o, sf = wkv7.gdn_fwd_varlen(*(dev[n] for n in NAMES), torch.from_numpy(cu).cuda(),
                                initial_state=torch.from_numpy(poolv).cuda(),
                                state_map=None if smap is None else torch.from_numpy(smap).cuda(), algo=algo)
    torch.cuda.synchronize()
    o, sf = hz.to_np(o), hz.to_np(sf)
    for n in range(N):
        s_, e_ = int(cu[n]), int(cu[n + 1])
        row = {"map": None if smap is None else int(smap[n]), "shared": 0, "rows": n}[pool]
        s0 = poolv[row:row + 1] if row is not None and 0 <= row < n_pool else None
        sl = {x: inp[x][:, s_:e_] for x in NAMES}
        o_ref, s_ref = oracle.gdn_fwd(*(sl[x] for x in NAMES), s0)
        if e_ > s_:
            hz.check("bf16", o[s_:e_], o_ref[0], sf[n], s_ref[0], what=f"gdn varlen D{D} seq{n}")
        else:
            np.testing.assert_array_equal(sf[n], s_ref[0])


@pytest.mark.parametrize("N", [128, 129])
def test_gdn_varlen_many_sequences_with_equal_lengths(N):
    """Many packed Gated DeltaNet sequences with repeated lengths (ties in
    the chunked kernel's longest-first order), at and just past the largest
    count that order covers: every sequence against the oracle."""
    rng = np.random.default_rng(4950 + N)
    lengths = rng.choice([0, 1, 16, 400, 517, 600, 700], size=N).tolist()
    assert N > 128 or sum(lengths) >= 256 * N   # the longest-first order applies
    TT, H, D = sum(lengths), 3, 64
    inp = synth.make_gdn(1, TT, H, D, seed=4951 + N, init=False)
    poolv = (rng.standard_normal((3, H, D, D)) * 0.1).astype(np.float32)
    smap = rng.integers(-1, 4, size=N).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = {n: synth.to_torch(inp[n][0], "bf16", "cuda") for n in NAMES}
    o, sf = wkv7.gdn_fwd_varlen(*(dev[n] for n in NAMES), torch.from_numpy(cu).cuda(),
                                initial_state=torch.from_numpy(poolv).cuda(), state_map=torch.from_numpy(smap).cuda(),
                                algo=CHK)
    torch.cuda.synchronize()
    o, sf = hz.to_np(o), hz.to_np(sf)
    for n in range(N):
        s_, e_ = int(cu[n]), int(cu[n + 1])
        row = int(smap[n])
        s0 = poolv[row:row + 1] if 0 <= row < 3 else None
        sl = {x: inp[x][:, s_:e_] for x in NAMES}
        o_ref, s_ref = oracle.gdn_fwd(*(sl[x] for x in NAMES), s0)
        if e_ > s_:
            hz.check("bf16", o[s_:e_], o_ref[0], sf[n], s_ref[0], what=f"gdn varlen N={N} seq{n}")
        else:
            np.testing.assert_array_equal(sf[n], s_ref[0])

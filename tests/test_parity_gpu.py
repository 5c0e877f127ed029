"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Inputs come from the seeded generator shared by both sides; the oracle sees
exactly the values the GPU sees (already rounded to the I/O dtype).  Every case
is compared element by element over every output, the full-size workloads
included (every (b, h) sequence, each against its own output RMS).
"""
import numpy as np
import pytest

import harness as hz
import oracle
from rwkv_linear_attention_amd import synth, wkv7

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REC, CHK = wkv7.ALGO_RECURRENT, wkv7.ALGO_CHUNKED


def run_case(inp, algo, what):
    dev = hz.to_dev(inp)
    o, sf = hz.gpu_fwd(dev, algo=algo)
    torch.cuda.synchronize()
    o_ref, s_ref = hz.oracle_fwd(inp)
    return hz.check(inp["dtype"], hz.to_np(o), o_ref, hz.to_np(sf), s_ref, what)


# ---- the named workloads ------------------------------------------------------

@pytest.mark.parametrize("algo", [REC, CHK, wkv7.ALGO_AUTO])
def test_workload0_fp32_full(algo):
    run_case(synth.make(0), algo, f"workload 0 algo {algo}")


@pytest.mark.parametrize("algo", [REC, CHK, wkv7.ALGO_AUTO])
def test_workload1_bf16_mask_state_full(algo):
    run_case(synth.make(1), algo, f"workload 1 algo {algo}")


def sampled_pairs(B, H):
    pairs = {(0, 0), (B - 1, H - 1), (0, H - 1), (B - 1, 0), (B // 2, H // 2), (1 % B, 3 % H)}
    return sorted(pairs)


@pytest.mark.parametrize("idx", [2, 3])
def test_full_size_workload_all_sequences(idx):
    """Full-size workloads in the launch configuration the benchmark times
    (ALGO_AUTO -> chunked kernel): o and the final state of every (b, h)
    sequence against the oracle (one OpenMP pass over all sequences)."""
    inp = synth.make(idx)
    B, T, H, D = inp["r"].shape
    assert wkv7.fwd_path(torch.bfloat16, B, T, H, D, D) == CHK
    dev = hz.to_dev(inp)
    o, sf = hz.gpu_fwd(dev)
    torch.cuda.synchronize()
    del dev
    o_ref, s_ref = hz.oracle_fwd(inp)
    wo, ws = hz.check_sequences("bf16", o, o_ref, sf, s_ref, f"workload {idx} all sequences")
    print(f"workload {idx}: worst output ratio {wo:.3f}, worst state ratio {ws:.3f}")


@pytest.mark.parametrize("algo", [wkv7.ALGO_AUTO, REC])
def test_full_size_fp32_all_sequences(algo):
    """The workload-2 shape (B8 T4096 H64 d64) with fp32 I/O: under AUTO
    (the fp32 chunked kernel, as the benchmark times it) and on the
    recurrent kernel; every sequence against the fp32 rule (max-abs 1e-4 on
    o and the final state)."""
    inp = dict(synth.make(2), dtype="f32")
    B, T, H, D = inp["r"].shape
    if algo == wkv7.ALGO_AUTO:
        assert wkv7.fwd_path(torch.float32, B, T, H, D, D) == CHK
    dev = hz.to_dev(inp)
    o, sf = hz.gpu_fwd(dev, algo=algo)
    torch.cuda.synchronize()
    del dev
    o_ref, s_ref = hz.oracle_fwd(inp)
    wo, ws = hz.check_sequences("f32", o, o_ref, sf, s_ref, f"fp32 workload-2 shape algo {algo} all sequences")
    print(f"fp32 B8 T4096 H64 d64 algo {algo}: worst output ratio {wo:.3f}, worst state ratio {ws:.3f}")


def test_full_size_fp32_d128_all_sequences():
    """The workload-3 shape (B16 T4096 H32 d128, initial state, trailing
    padding) with fp32 I/O under AUTO (fp32 chunked kernel), every sequence."""
    inp = dict(synth.make(3), dtype="f32")
    B, T, H, D = inp["r"].shape
    assert wkv7.fwd_path(torch.float32, B, T, H, D, D) == CHK
    dev = hz.to_dev(inp)
    o, sf = hz.gpu_fwd(dev)
    torch.cuda.synchronize()
    del dev
    o_ref, s_ref = hz.oracle_fwd(inp)
    wo, ws = hz.check_sequences("f32", o, o_ref, sf, s_ref, "fp32 workload-3 shape all sequences")
    print(f"fp32 B16 T4096 H32 d128: worst output ratio {wo:.3f}, worst state ratio {ws:.3f}")


def test_workload4_decode_steps_all_sequences():
    """256 consecutive wkv7_step calls on B=512, H=40, d=64 (state in
    place).  Every output of every step and all 20480 final states are
    compared with the oracle's forward over the same 256 tokens (a step loop
    equals the forward, pinned on the oracle); two sequences are also
    replayed step by step through the oracle's own step function."""
    inp = synth.make(4)
    B, T, H, D = inp["r"].shape
    dev = hz.to_dev(inp)
    state = dev["s0"].clone()
    o_all = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        o_all[:, t] = wkv7.step(*(dev[n][:, t].contiguous() for n in hz.ARRAYS), state)
    torch.cuda.synchronize()
    o_ref, s_ref = hz.oracle_fwd(inp)
    wo, ws = hz.check_sequences("bf16", o_all, o_ref, state, s_ref, "decode 256 steps all sequences")
    print(f"decode: worst output ratio {wo:.3f}, worst state ratio {ws:.3f}")
    for bb, h in ((0, 0), (B - 1, H - 1)):
        S = inp["s0"][bb:bb + 1, h:h + 1].astype(np.float64)
        o_step = np.zeros((T, D))
        for t in range(T):
            sl = lambda n: inp[n][bb:bb + 1, t, h:h + 1]
            ot, S = oracle.step(sl("r"), sl("w"), sl("k"), sl("v"), sl("a"), sl("b"), S)
            o_step[t] = ot[0, 0]
        hz.check("bf16", hz.to_np(o_all[bb, :, h]), o_step, hz.to_np(state[bb, h]), S[0, 0],
                 f"decode step oracle (b={bb}, h={h})")


# ---- shapes, tails and both kernels -----------------------------------------

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 65, 1000])
@pytest.mark.parametrize("algo", [REC, CHK])
def test_shapes_bf16(D, T, algo):
    inp = synth.make(1, B=1, T=T, H=3, K=D, seed=7 * T + D)
    run_case(inp, algo, f"D={D} T={T} algo={algo}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 200, 1000])
@pytest.mark.parametrize("algo", [REC, CHK])
def test_shapes_fp32(D, T, algo):
    wl = dict(synth.WORKLOADS[0], dtype="f32")
    inp = synth.make(wl, B=3, T=T, H=2, K=D, seed=11 * T + D, init=True, mask="bernoulli")
    run_case(inp, algo, f"fp32 D={D} T={T} algo={algo}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["zeros", "trailing", "leading", "nonfinite_masked", "extreme_decay", "no_state"])
def test_fp32_chunked_cases(D, kind):
    """The fp32 chunked kernel on masks, non-finite inputs at masked tokens,
    chunks that need the exact token-by-token path, and no initial state."""
    wl = dict(synth.WORKLOADS[0], dtype="f32")
    B, T, H = 2, 100, 2
    inp = synth.make(wl, B=B, T=T, H=H, K=D, seed=900 + D, init=kind != "no_state", mask="bernoulli")
    if kind == "zeros":
        inp["mask"] = np.zeros((B, T), np.uint8)
    elif kind == "trailing":
        inp["mask"] = np.ones((B, T), np.uint8)
        inp["mask"][:, 83:] = 0
    elif kind == "leading":
        inp["mask"] = np.ones((B, T), np.uint8)
        inp["mask"][:, :37] = 0
    elif kind == "extreme_decay":
        w = inp["w"].copy()
        w[:, 20] = -1e9
        w[1, 55, :, :8] = -1e9
        w[0, 70, 1, 3] = 0.05
        w[0, 80:96] = -20.0
        inp["w"] = w
    o_ref, s_ref = hz.oracle_fwd(inp)
    if kind == "nonfinite_masked":
        masked = inp["mask"] == 0
        for n, val in zip("wkvab", (np.nan, np.inf, np.nan, -np.inf, np.nan)):
            x = np.array(inp[n], copy=True)
            x[masked] = val
            inp[n] = x
    dev = hz.to_dev(inp)
    o, sf = hz.gpu_fwd(dev, algo=CHK)
    torch.cuda.synchronize()
    hz.check("f32", hz.to_np(o), o_ref, hz.to_np(sf), s_ref, f"fp32 chunked {kind} D={D}")
    if kind == "zeros":
        assert torch.equal(sf, dev["s0"]), "all-masked sequence must leave the state bit-exact"


@pytest.mark.parametrize("D", [64, 128])
def test_fp32_chunked_equals_recurrent(D):
    inp = synth.make(dict(synth.WORKLOADS[0], dtype="f32"), B=2, T=300, H=2, K=D, seed=97 + D, init=True,
                     mask="bernoulli")
    dev = hz.to_dev(inp)
    o1, s1 = hz.gpu_fwd(dev, algo=REC)
    o2, s2 = hz.gpu_fwd(dev, algo=CHK)
    torch.cuda.synchronize()
    o_ref, s_ref = hz.oracle_fwd(inp)
    hz.check("f32", hz.to_np(o1), o_ref, hz.to_np(s1), s_ref, "fp32 recurrent")
    hz.check("f32", hz.to_np(o2), o_ref, hz.to_np(s2), s_ref, "fp32 chunked")
    hz.check("f32", hz.to_np(o2), hz.to_np(o1), hz.to_np(s2), hz.to_np(s1), "fp32 chunked vs recurrent",
             scale=2.0)


@pytest.mark.parametrize("D", [64, 128])
def test_chunked_equals_recurrent(D):
    """Both GPU kernels agree on the same inputs, and each agrees with the oracle."""
    inp = synth.make(1, B=2, T=300, H=2, K=D, seed=99 + D)
    dev = hz.to_dev(inp)
    o1, s1 = hz.gpu_fwd(dev, algo=REC)
    o2, s2 = hz.gpu_fwd(dev, algo=CHK)
    torch.cuda.synchronize()
    o_ref, s_ref = hz.oracle_fwd(inp)
    hz.check("bf16", hz.to_np(o1), o_ref, hz.to_np(s1), s_ref, "recurrent")
    hz.check("bf16", hz.to_np(o2), o_ref, hz.to_np(s2), s_ref, "chunked")
    hz.check("bf16", hz.to_np(o2), hz.to_np(o1), hz.to_np(s2), hz.to_np(s1), "chunked vs recurrent", scale=2.0)


# ---- masks and state handling ------------------------------------------------

@pytest.mark.parametrize("algo", [REC, CHK])
@pytest.mark.parametrize("kind", ["zeros", "ones", "bernoulli", "trailing", "leading"])
def test_masks(algo, kind):
    inp = synth.make(1, B=3, T=100, H=2, K=64, seed=5)
    B, T = 3, 100
    if kind == "zeros":
        inp["mask"] = np.zeros((B, T), np.uint8)
    elif kind == "ones":
        inp["mask"] = np.ones((B, T), np.uint8)
    elif kind == "trailing":
        inp["mask"] = np.ones((B, T), np.uint8)
        inp["mask"][:, 77:] = 0
    elif kind == "leading":
        inp["mask"] = np.ones((B, T), np.uint8)
        inp["mask"][:, :40] = 0
    run_case(inp, algo, f"mask {kind} algo {algo}")
    if kind == "zeros":
        dev = hz.to_dev(inp)
        _, sf = hz.gpu_fwd(dev, algo=algo)
        assert torch.equal(sf, dev["s0"]), "all-masked sequence must leave the state bit-exact"


@pytest.mark.parametrize("D", [64, 128])
def test_chunked_deterministic_many_sequences(D):
    """Repeated launches give bit-identical outputs and states.  The kernel's
    arithmetic has no atomics or order-dependent reductions, so any difference
    means a hand-off race between producer and consumer waves; enough
    sequences run at once here to fill every CU."""
    H = 4096 // D
    inp = synth.make(1, B=8, T=1024, H=H, K=D, seed=31 + D, init=True, mask="bernoulli")
    dev = hz.to_dev(inp)
    o0, s0 = hz.gpu_fwd(dev, algo=CHK)
    for _ in range(4):
        o1, s1 = hz.gpu_fwd(dev, algo=CHK)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(s0, s1), "chunked forward is not deterministic"
    # and the first sequence still matches the oracle
    (o_ref, s_ref), = hz.oracle_fwd(inp, bh=[(3, H - 1)])
    hz.check("bf16", hz.to_np(o0[3, :, H - 1]), o_ref, hz.to_np(s0[3, H - 1]), s_ref, f"deterministic D={D}")


@pytest.mark.parametrize("algo", [REC, CHK])
@pytest.mark.parametrize("D", [64, 128])
def test_masked_tokens_ignore_nonfinite_inputs(algo, D):
    """A masked token leaves the state alone whatever its w, k, v, a, b hold
    (padding may be uninitialised memory); its r still produces an output."""
    inp = synth.make(1, B=2, T=100, H=2, K=D, seed=21 + D, init=True, mask="bernoulli")
    o_ref, s_ref = hz.oracle_fwd(inp)
    bad = dict(inp)
    masked = inp["mask"] == 0
    assert masked.any() and (~masked).any()
    for n, val in zip("wkvab", (np.nan, np.inf, np.nan, -np.inf, np.nan)):
        x = np.array(inp[n], copy=True)
        x[masked] = val
        bad[n] = x
    o, sf = hz.gpu_fwd(hz.to_dev(bad), algo=algo)
    torch.cuda.synchronize()
    hz.check("bf16", hz.to_np(o), o_ref, hz.to_np(sf), s_ref, f"non-finite masked tokens D={D} algo={algo}")


@pytest.mark.parametrize("algo", [REC, CHK])
def test_state_aliasing_and_null_states(algo):
    inp = synth.make(1, B=2, T=70, H=2, K=64, seed=3)
    dev = hz.to_dev(inp)
    o_ref, s_ref = hz.oracle_fwd(inp)
    # final_state aliasing initial_state
    st = dev["s0"].clone()
    o, sf = wkv7.fwd(*(dev[n] for n in hz.ARRAYS), initial_state=st, mask=dev["mask"],
                     algo=algo, final_state=st)
    torch.cuda.synchronize()
    assert sf.data_ptr() == st.data_ptr()
    hz.check("bf16", hz.to_np(o), o_ref, hz.to_np(st), s_ref, "aliased state")
    # NULL initial state equals an explicit zero state
    z = torch.zeros_like(dev["s0"])
    o1, s1 = wkv7.fwd(*(dev[n] for n in hz.ARRAYS), initial_state=None, mask=dev["mask"], algo=algo)
    o2, s2 = wkv7.fwd(*(dev[n] for n in hz.ARRAYS), initial_state=z, mask=dev["mask"], algo=algo)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    # NULL final state: output unchanged, nothing else written
    o3, s3 = wkv7.fwd(*(dev[n] for n in hz.ARRAYS), initial_state=None, mask=dev["mask"],
                      algo=algo, output_final_state=False)
    assert s3 is None and torch.equal(o3, o1)


def test_state_passing_composition():
    """fwd over [0, T) equals fwd over [T1, T) from fwd([0, T1)).final."""
    inp = synth.make(1, B=2, T=160, H=2, K=64, seed=8)
    dev = hz.to_dev(inp)
    o, sf = hz.gpu_fwd(dev, algo=CHK)
    T1 = 48
    part = lambda lo, hi: {n: dev[n][:, lo:hi].contiguous() for n in hz.ARRAYS}
    p1, p2 = part(0, T1), part(T1, 160)
    m1 = dev["mask"][:, :T1].contiguous()
    m2 = dev["mask"][:, T1:].contiguous()
    oa, sa = wkv7.fwd(*(p1[n] for n in hz.ARRAYS), initial_state=dev["s0"], mask=m1, algo=CHK)
    ob, sb = wkv7.fwd(*(p2[n] for n in hz.ARRAYS), initial_state=sa, mask=m2, algo=CHK)
    torch.cuda.synchronize()
    o_ref, s_ref = hz.oracle_fwd(inp)
    hz.check("bf16", hz.to_np(torch.cat([oa, ob], 1)), o_ref, hz.to_np(sb), s_ref, "composed")


def test_empty_sequence():
    inp = synth.make(1, B=2, T=1, H=2, K=64, seed=1)
    dev = hz.to_dev(inp)
    empty = {n: dev[n][:, :0].contiguous() for n in hz.ARRAYS}
    o, sf = wkv7.fwd(*(empty[n] for n in hz.ARRAYS), initial_state=dev["s0"])
    o2, sf2 = wkv7.fwd(*(empty[n] for n in hz.ARRAYS), initial_state=None)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64)
    assert torch.equal(sf, dev["s0"]) and torch.count_nonzero(sf2) == 0


@pytest.mark.parametrize("algo", [REC, CHK])
def test_extreme_decay_tokens(algo):
    """w = -1e9 on some tokens (a full reset of those channels) and a few
    positive w: the chunked kernel must take its exact path; outputs stay
    finite and match the oracle."""
    inp = synth.make(1, B=2, T=90, H=2, K=64, seed=21)
    rng = np.random.default_rng(0)
    w = inp["w"].copy()
    w[:, 20] = -1e9
    w[1, 55, :, :8] = -1e9
    w[0, 70, 1, 3] = 0.05
    inp["w"] = synth.round_to(w, "bf16")
    run_case(inp, algo, f"extreme decay algo {algo}")


@pytest.mark.parametrize("algo", [REC, CHK])
def test_outputs_fully_written_and_guarded(algo):
    """NaN-prefilled output and guard bands around o and the final state:
    every output element is written and nothing outside is touched."""
    inp = synth.make(1, B=2, T=37, H=3, K=64, seed=4)
    dev = hz.to_dev(inp)
    B, T, H, D = 2, 37, 3, 64
    n_o = B * T * H * D
    guard = 1024
    obuf = torch.full((n_o + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    sbuf = torch.full((B * H * D * D + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[guard:guard + n_o].view(B, T, H, D)
    s = sbuf[guard:guard + B * H * D * D].view(B, H, D, D)
    wkv7.fwd(*(dev[n] for n in hz.ARRAYS), initial_state=dev["s0"], mask=dev["mask"], algo=algo,
             out=o, final_state=s)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all()
    assert torch.isnan(obuf[:guard].float()).all() and torch.isnan(obuf[-guard:].float()).all()
    assert torch.isnan(sbuf[:guard]).all() and torch.isnan(sbuf[-guard:]).all()


def test_step_matches_forward_and_oracle():
    """T consecutive decode steps equal the forward over T tokens (d=64 and 128)."""
    for D in (64, 128):
        inp = synth.make(1, B=3, T=12, H=2, K=D, seed=D, mask="none")
        dev = hz.to_dev(inp)
        o_f, s_f = hz.gpu_fwd(dev, algo=REC)
        st = dev["s0"].clone()
        outs = [wkv7.step(*(dev[n][:, t].contiguous() for n in hz.ARRAYS), st) for t in range(12)]
        torch.cuda.synchronize()
        o_ref, s_ref = hz.oracle_fwd(inp)
        hz.check("bf16", hz.to_np(torch.stack(outs, 1)), o_ref, hz.to_np(st), s_ref, f"step D={D}")
        hz.check("bf16", hz.to_np(o_f), o_ref, hz.to_np(s_f), s_ref, f"fwd D={D}")


def test_step_fp32():
    wl = dict(synth.WORKLOADS[4], dtype="f32")
    inp = synth.make(wl, B=4, T=3, H=5, K=64, seed=77)
    dev = hz.to_dev(inp)
    st = dev["s0"].clone()
    outs = [wkv7.step(*(dev[n][:, t].contiguous() for n in hz.ARRAYS), st) for t in range(3)]
    torch.cuda.synchronize()
    o_ref, s_ref = hz.oracle_fwd(inp)
    hz.check("f32", hz.to_np(torch.stack(outs, 1)), o_ref, hz.to_np(st), s_ref, "step fp32")

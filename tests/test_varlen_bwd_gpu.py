"""GPU parity of wkv7_bwd_varlen (gradients over packed variable-length
sequences) against the fp64 backward oracle run on each sequence alone: by
definition each packed sequence is an independent run from the pool row its
state_map entry names (an index outside the pool means a zero state).
Tolerances are those of tests/test_bwd_gpu.py."""
import numpy as np
import pytest

import harness as hz
import oracle
from rwkv_linear_attention_amd import synth, wkv7
from harness import check_grad

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("r", "w", "k", "v", "a", "b")


def packed_case(lengths, H, D, dtype, seed, n_state=None, smap=None, masked=True):
    TT = int(sum(lengths))
    inp = synth.make(1, B=1, T=max(TT, 1), H=H, K=D, seed=seed, init=False, mask="bernoulli" if masked else "none")
    x = {n: synth.round_to(inp[n][0, :TT], dtype) for n in NAMES}
    mask = inp["mask"][0, :TT] if masked else None
    rng = np.random.default_rng(seed + 3)
    N = len(lengths)
    pool = None if n_state is None else (rng.standard_normal((n_state, H, D, D)) * 0.1).astype(np.float32)
    d_o = synth.round_to(rng.standard_normal((TT, H, D)).astype(np.float32), dtype)
    d_sf = (rng.standard_normal((N, H, D, D)) * 0.5).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return dict(x=x, mask=mask, pool=pool, smap=smap, d_o=d_o, d_sf=d_sf, cu=cu, dtype=dtype)


def run_gpu(c):
    dt = c["dtype"]
    dev = {n: synth.to_torch(c["x"][n], dt, "cuda") for n in NAMES}
    t = lambda a, dtype=None: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    g = wkv7.bwd_varlen(*(dev[n] for n in NAMES), t(c["cu"]), synth.to_torch(c["d_o"], dt, "cuda"),
                        initial_state=t(c["pool"]), state_map=t(c["smap"]), mask=t(c["mask"]),
                        d_final_state=t(c["d_sf"]))
    torch.cuda.synchronize()
    return {n: hz.to_np(v) for n, v in g.items()}


def check_against_oracle(c, g, what, vanishing_floor=False):
    cu, dt = c["cu"], c["dtype"]
    for n in range(len(cu) - 1):
        tb, te = int(cu[n]), int(cu[n + 1])
        s0 = None
        if c["pool"] is not None:
            row = n if c["smap"] is None else int(c["smap"][n])
            if 0 <= row < c["pool"].shape[0]:
                s0 = c["pool"][row][None]
        if te == tb:
            np.testing.assert_array_equal(g["s0"][n], c["d_sf"][n])
            continue
        sl = {k: c["x"][k][tb:te][None] for k in NAMES}
        m = None if c["mask"] is None else c["mask"][tb:te][None]
        ref = oracle.bwd(*(sl[k] for k in NAMES), c["d_o"][tb:te][None], s0, m, c["d_sf"][n][None])
        fl = float(np.sqrt(np.mean(np.concatenate([ref[k].ravel() for k in NAMES]) ** 2))) if vanishing_floor else 0.0
        for k in NAMES:
            check_grad(dt, g[k][tb:te], ref[k][0], f"{what} seq{n} d{k}", floor=fl)
        check_grad("f32", g["s0"][n], ref["s0"][0], f"{what} seq{n} ds0")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64), ("bf16", 128), ("f32", 128)])
def test_bwd_varlen_parity_pool_and_map(dtype, D):
    lengths = [0, 1, 17, 50, 33, 130] if D == 64 else [40, 0, 25, 16]
    smap = np.array([2, 0, -1, 1, 2, 5][:len(lengths)], np.int32)   # -1 and 5: zero state
    c = packed_case(lengths, 2, D, dtype, seed=9100 + D, n_state=3, smap=smap)
    check_against_oracle(c, run_gpu(c), f"bwd varlen {dtype} D{D}")


def test_bwd_varlen_one_row_per_sequence_no_mask():
    c = packed_case([33, 64, 7], 3, 64, "bf16", seed=9200, n_state=3, smap=None, masked=False)
    check_against_oracle(c, run_gpu(c), "bwd varlen rows")


def test_bwd_varlen_equal_lengths_match_fixed_length():
    """B sequences of one length packed back to back give exactly the
    fixed-length backward's gradients (same kernels, same chunking)."""
    B, T, H, D = 3, 70, 2, 64
    inp = synth.make(1, B=B, T=T, H=H, K=D, seed=9300, init=True, mask="bernoulli")
    dev = {n: synth.to_torch(inp[n], "bf16", "cuda") for n in NAMES}
    rng = np.random.default_rng(9301)
    d_o = synth.to_torch(synth.round_to(rng.standard_normal((B, T, H, D)).astype(np.float32), "bf16"), "bf16", "cuda")
    s0 = torch.from_numpy(inp["s0"]).cuda()
    mask = torch.from_numpy(inp["mask"]).cuda()
    fixed = wkv7.bwd(*(dev[n] for n in NAMES), d_o, initial_state=s0, mask=mask)
    cu = torch.arange(0, (B + 1) * T, T, dtype=torch.int32, device="cuda")
    flat = lambda t: t.reshape(B * T, H, D)
    packed = wkv7.bwd_varlen(*(flat(dev[n]) for n in NAMES), cu, flat(d_o), initial_state=s0,
                             mask=mask.reshape(B * T))
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(packed[n].reshape(B, T, H, D), fixed[n]), n
    assert torch.equal(packed["s0"], fixed["s0"])


def test_bwd_varlen_all_empty():
    c = packed_case([0, 0, 0], 1, 64, "bf16", seed=9400, masked=False)
    g = run_gpu(c)
    np.testing.assert_array_equal(g["s0"], c["d_sf"])


def test_bwd_varlen_malformed_offsets_stay_in_bounds():
    """Offsets that decrease make sequences overlap, so their chunk count
    exceeds the workspace's capacity: the call still returns normally (the
    offsets are clamped and the checkpoint storage saturates), and the first
    sequence, which precedes the overlap in chunk order, is still right."""
    H, D = 1, 64
    c = packed_case([64], H, D, "bf16", seed=9500, masked=False)
    c["cu"] = np.array([0, 64, 0, 64, 0, 64], np.int32)   # N = 5: 4 + 0 + 4 + 0 + 4 chunks > capacity 9
    c["d_sf"] = np.zeros((5, H, D, D), np.float32)
    g = run_gpu(c)
    assert np.all(np.isfinite(g["s0"]))
    ref = oracle.bwd(*(c["x"][k][None] for k in NAMES), c["d_o"][None], None, None, None)
    check_grad("f32", g["s0"][0], ref["s0"][0], "bwd varlen malformed seq0 ds0")


@pytest.mark.parametrize("N", [128, 129])
def test_bwd_varlen_many_sequences_with_equal_lengths(N):
    """Many packed sequences with repeated lengths (ties in the recurrences'
    longest-first order, taken by packed calls of at most 128 sequences
    averaging at least 256 tokens), at and just past the largest count that
    order covers (above it the index order): every sequence's gradients
    against the oracle."""
    rng = np.random.default_rng(9300 + N)
    lengths = rng.choice([0, 1, 17, 400, 517, 600, 700], size=N).tolist()
    assert N > 128 or sum(lengths) >= 256 * N
    smap = rng.integers(-1, 4, size=N).astype(np.int32)
    c = packed_case(lengths, 2, 64, "bf16", seed=9301 + N, n_state=3, smap=smap)
    # one-token sequences from a zero state have dw = 0 identically: the
    # documented floor (the call's gradient RMS) applies to those alone
    check_against_oracle(c, run_gpu(c), f"bwd varlen N={N}", vanishing_floor=True)


def test_bwd_varlen_longest_first_malformed_offsets_stay_in_bounds():
    """The same saturation under the recurrences' longest-first order (3
    sequences averaging 341 tokens, overlapping): the call returns
    normally with finite state gradients, and the first sequence, whose
    checkpoints precede the overlap in chunk order, is still right."""
    H, D = 1, 64
    c = packed_case([1024], H, D, "bf16", seed=9510, masked=False)
    c["cu"] = np.array([0, 1024, 0, 1024], np.int32)   # 64 + 0 + 64 chunks > capacity 67
    c["d_sf"] = np.zeros((3, H, D, D), np.float32)
    g = run_gpu(c)
    assert np.all(np.isfinite(g["s0"]))
    ref = oracle.bwd(*(c["x"][k][None] for k in NAMES), c["d_o"][None], None, None, None)
    check_grad("f32", g["s0"][0], ref["s0"][0], "bwd varlen malformed (longest first) seq0 ds0")

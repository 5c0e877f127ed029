"""GPU parity of wkv7_fwd_varlen (packed variable-length sequences with a
state_map into a pool of initial states) against the fp64 oracle.

Each packed sequence is, by definition, an independent run of the operator
(rwkv-fla page, news note on variable-length inputs; rwkv-ops README,
state_map of the operator interface), so the expected values come from the
oracle run on each sequence's slice with its mapped initial state.
"""
import numpy as np
import pytest

import harness as hz
from rwkv_linear_attention_amd import synth, wkv7

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REC, CHK = wkv7.ALGO_RECURRENT, wkv7.ALGO_CHUNKED


def packed_case(lengths, H, D, seed, n_state, state_map, mask=True):
    """Draw one packed batch: the synthetic recipe on a [1, T_total, H, D]
    axis, a pool of n_state initial states and an optional Bernoulli mask."""
    TT = int(sum(lengths))
    inp = synth.make(1, B=1, T=max(TT, 1), H=H, K=D, seed=seed, init=False,
                     mask="bernoulli" if mask else "none")
    rng = np.random.default_rng(seed + 1)
    pool = (rng.standard_normal((n_state, H, D, D)) * 0.1).astype(np.float32) if n_state else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    arrs = {n: inp[n][0, :TT] for n in "rwkvab"}
    m = inp["mask"][0, :TT] if mask else None
    return arrs, cu, pool, None if state_map is None else np.asarray(state_map, np.int32), m


def oracle_varlen(arrs, cu, pool, smap, m, H, D):
    outs, states = [], []
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        idx = n if smap is None else int(smap[n])
        s0 = None if pool is None or not (0 <= idx < pool.shape[0]) else pool[idx:idx + 1]
        inp = {x: arrs[x][None, s:e] for x in "rwkvab"}
        inp["s0"] = s0
        inp["mask"] = None if m is None else m[None, s:e]
        o, sf = hz.oracle_fwd(inp)
        outs.append(o[0])
        states.append(sf[0])
    return outs, states


def run_gpu(arrs, cu, pool, smap, m, algo):
    dev = {x: synth.to_torch(arrs[x], "bf16", "cuda") for x in "rwkvab"}
    cu_t = torch.from_numpy(cu).cuda()
    pool_t = None if pool is None else torch.from_numpy(pool).cuda()
    smap_t = None if smap is None else torch.from_numpy(smap).cuda()
    m_t = None if m is None else torch.from_numpy(m).cuda()
    o, sf = wkv7.fwd_varlen(*(dev[x] for x in "rwkvab"), cu_t, initial_state=pool_t, state_map=smap_t,
                            mask=m_t, algo=algo)
    torch.cuda.synchronize()
    return hz.to_np(o), hz.to_np(sf)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("algo", [REC, CHK])
def test_varlen_mixed_lengths_and_state_map(D, algo):
    lengths = [17, 0, 1, 100, 15, 16, 333, 2]
    smap = [2, -1, 0, 1, 2, 7, 0, 1]          # -1 and 7 are out of range: zero state
    arrs, cu, pool, smap, m = packed_case(lengths, H=3, D=D, seed=41 + D, n_state=3, state_map=smap)
    o, sf = run_gpu(arrs, cu, pool, smap, m, algo)
    outs, states = oracle_varlen(arrs, cu, pool, smap, m, H=3, D=D)
    for n in range(len(lengths)):
        s, e = int(cu[n]), int(cu[n + 1])
        if e > s:
            hz.check("bf16", o[s:e], outs[n], sf[n], states[n], f"varlen seq {n} (T={e - s}) D={D} algo={algo}")
        else:
            exp = np.zeros_like(sf[n]) if not (0 <= smap[n] < 3) else pool[smap[n]]
            assert np.array_equal(sf[n], exp), f"empty sequence {n} must return its initial state"


@pytest.mark.parametrize("D", [64, 128])
def test_varlen_equal_lengths_match_fixed_length_call(D):
    """Equal lengths and no state_map reproduce wkv7_fwd bit for bit."""
    B, T, H = 3, 80, 2
    inp = synth.make(1, B=B, T=T, H=H, K=D, seed=53, init=True, mask="bernoulli")
    dev = hz.to_dev(inp)
    o1, s1 = hz.gpu_fwd(dev, algo=CHK)
    flat = {x: dev[x].reshape(B * T, H, D) for x in "rwkvab"}
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
    o2, s2 = wkv7.fwd_varlen(*(flat[x] for x in "rwkvab"), cu, initial_state=dev["s0"],
                             mask=dev["mask"].reshape(B * T), algo=CHK)
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(B * T, H, D), o2) and torch.equal(s1, s2)


def test_varlen_shared_state_and_empty_axis():
    """n_state = 1 shares one initial state; an all-empty batch returns the
    mapped initial states unchanged."""
    D, H = 64, 2
    arrs, cu, pool, smap, m = packed_case([40, 23, 64], H=H, D=D, seed=61, n_state=1, state_map=[0, 0, 0])
    o, sf = run_gpu(arrs, cu, pool, smap, m, CHK)
    outs, states = oracle_varlen(arrs, cu, pool, smap, m, H=H, D=D)
    for n in range(3):
        s, e = int(cu[n]), int(cu[n + 1])
        hz.check("bf16", o[s:e], outs[n], sf[n], states[n], f"shared-state seq {n}")
    # all sequences empty
    z = torch.zeros((0, H, D), dtype=torch.bfloat16, device="cuda")
    cu0 = torch.zeros(4, dtype=torch.int32, device="cuda")
    pool_t = torch.from_numpy(np.random.default_rng(3).standard_normal((2, H, D, D)).astype(np.float32)).cuda()
    smap_t = torch.tensor([1, 0, 5], dtype=torch.int32, device="cuda")
    o0, s0 = wkv7.fwd_varlen(z, z, z, z, z, z, cu0, initial_state=pool_t, state_map=smap_t)
    torch.cuda.synchronize()
    assert o0.shape == (0, H, D)
    assert torch.equal(s0[0], pool_t[1]) and torch.equal(s0[1], pool_t[0]) and torch.all(s0[2] == 0)


@pytest.mark.parametrize("N", [128, 129])
def test_varlen_many_sequences_with_equal_lengths(N):
    """Many packed sequences with repeated lengths (ties in the chunked
    kernel's longest-first order, which packed calls of at most 128
    sequences averaging at least 256 tokens take), at and just past the
    largest count that order covers (above it the workgroups take the
    sequences in index order): every sequence against the oracle."""
    rng = np.random.default_rng(70 + N)
    lengths = rng.choice([0, 1, 16, 400, 517, 600, 700], size=N).tolist()
    assert N > 128 or sum(lengths) >= 256 * N
    smap = rng.integers(-1, 4, size=N).tolist()
    arrs, cu, pool, smap, m = packed_case(lengths, H=3, D=64, seed=71 + N, n_state=3, state_map=smap)
    o, sf = run_gpu(arrs, cu, pool, smap, m, CHK)
    outs, states = oracle_varlen(arrs, cu, pool, smap, m, H=3, D=64)
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        if e > s:
            hz.check("bf16", o[s:e], outs[n], sf[n], states[n], f"N={N} seq {n} (T={e - s})")
        else:
            exp = np.zeros_like(sf[n]) if not (0 <= smap[n] < 3) else pool[smap[n]]
            assert np.array_equal(sf[n], exp), f"empty sequence {n} must return its initial state"


@pytest.mark.parametrize("D", [64, 128])
def test_varlen_f32_chunked_mixed_and_equal_lengths(D):
    """fp32 I/O on the fp32 chunked kernel over packed sequences of mixed and
    repeated lengths averaging over 256 tokens (its longest-first order),
    each against the oracle at the fp32 bound."""
    lengths = [300, 0, 517, 300, 1, 700, 16, 517, 33]
    assert sum(lengths) >= 256 * len(lengths)
    smap = [2, -1, 0, 1, 2, 7, 0, 1, 1]
    arrs, cu, pool, smap, m = packed_case(lengths, H=3, D=D, seed=81 + D, n_state=3, state_map=smap)
    dev = {x: synth.to_torch(arrs[x], "f32", "cuda") for x in "rwkvab"}
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o, sf = wkv7.fwd_varlen(*(dev[x] for x in "rwkvab"), t(cu), initial_state=t(pool), state_map=t(smap),
                            mask=t(m), algo=CHK)
    torch.cuda.synchronize()
    o, sf = hz.to_np(o), hz.to_np(sf)
    outs, states = oracle_varlen(arrs, cu, pool, smap, m, H=3, D=D)
    for n in range(len(lengths)):
        s, e = int(cu[n]), int(cu[n + 1])
        if e > s:
            hz.check("f32", o[s:e], outs[n], sf[n], states[n], f"f32 varlen seq {n} (T={e - s}) D={D}")
        else:
            exp = np.zeros_like(sf[n]) if not (0 <= smap[n] < 3) else pool[smap[n]]
            assert np.array_equal(sf[n], exp), f"empty sequence {n} must return its initial state"


def test_varlen_longest_first_with_decreasing_offsets():
    """Decreasing offsets under the longest-first order (3 sequences
    averaging 400 tokens): lengths are clamped as in index order, so
    sequence 1 is empty and sequences 0 and 2 overlap on tokens 300..599.
    Each final state is that of its clamped range; outputs outside the
    overlap are those of the one sequence that covers them."""
    H, D, TT = 2, 64, 1200
    arrs, _, pool, _, m = packed_case([TT], H=H, D=D, seed=91, n_state=3, state_map=[0])
    cu = np.array([0, 600, 300, 1200], np.int32)
    smap = np.array([0, 1, 2], np.int32)
    o, sf = run_gpu(arrs, cu, pool, smap, m, CHK)
    ranges = [(0, 600), (600, 600), (300, 1200)]
    for n, (s, e) in enumerate(ranges):
        inp = {x: arrs[x][None, s:e] for x in "rwkvab"}
        inp["s0"] = pool[n:n + 1]
        inp["mask"] = m[None, s:e]
        if e == s:
            assert np.array_equal(sf[n], pool[n]), "an empty sequence returns its initial state"
            continue
        o_ref, s_ref = hz.oracle_fwd(inp)
        keep = slice(0, 300) if n == 0 else slice(300, 900)   # rows outside the overlap
        hz.check("bf16", o[s:e][keep], o_ref[0][keep], sf[n], s_ref[0], f"decreasing offsets seq {n}")

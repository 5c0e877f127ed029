"""GPU checks of the rwkv-ops-shaped entry points (api.py) against the fp64
oracle: gradients through torch.autograd equal the oracle's backward (tolerances
of tests/test_bwd_gpu.py), the inference twins return the same outputs
without a graph, and the one-token forms equal one step of the oracle."""
import numpy as np
import pytest

import harness as hz
import oracle
import rwkv_linear_attention_amd as m
from rwkv_linear_attention_amd import synth
from harness import check_grad

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("r", "w", "k", "v", "a", "b")
GNAMES = ("q", "k", "v", "g", "beta")


def leaf(x, dt):
    return synth.to_torch(x, dt, "cuda").requires_grad_(True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_generalized_delta_rule_autograd(dtype):
    B, T, H, D = 2, 70, 2, 64
    inp = synth.make(1, B=B, T=T, H=H, K=D, seed=8100, init=True, mask="bernoulli")
    for n in NAMES:
        inp[n] = synth.round_to(inp[n], dtype)
    rng = np.random.default_rng(8101)
    d_o = synth.round_to(rng.standard_normal((B, T, H, D)).astype(np.float32), dtype)
    d_sf = (rng.standard_normal((B, H, D, D)) * 0.5).astype(np.float32)
    x = {n: leaf(inp[n], dtype) for n in NAMES}
    s0 = torch.from_numpy(inp["s0"]).cuda().requires_grad_(True)
    mask = torch.from_numpy(inp["mask"]).cuda()
    o, sf = m.generalized_delta_rule(*(x[n] for n in NAMES), initial_state=s0, mask=mask)
    loss = (o.float() * synth.to_torch(d_o, "f32", "cuda")).sum() + (sf * torch.from_numpy(d_sf).cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd(*(inp[n] for n in NAMES), inp["s0"], inp["mask"])
    hz.check(dtype, hz.to_np(o), o_ref, hz.to_np(sf), s_ref, what=f"api gdr {dtype} o")
    ref = oracle.bwd(*(inp[n] for n in NAMES), d_o, inp["s0"], inp["mask"], d_sf)
    for n in NAMES:
        check_grad(dtype, hz.to_np(x[n].grad), ref[n], f"api gdr {dtype} d{n}")
    check_grad("f32", hz.to_np(s0.grad), ref["s0"], f"api gdr {dtype} ds0")
    # the gradient-free twin: same outputs, no graph
    o2, sf2 = m.generalized_delta_rule_inference(*(x[n] for n in NAMES), initial_state=s0, mask=mask)
    assert not o2.requires_grad
    np.testing.assert_array_equal(hz.to_np(o2), hz.to_np(o))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gated_delta_net_autograd_shared_state(dtype):
    B, T, H, D = 3, 48, 2, 64
    gi = synth.make_gdn(B, T, H, D, seed=8200, dtype=dtype, init=True, n_state=1)
    rng = np.random.default_rng(8201)
    d_o = synth.round_to(rng.standard_normal((B, T, H, D)).astype(np.float32), dtype)
    x = {n: leaf(gi[n], dtype) for n in GNAMES}
    s0 = torch.from_numpy(gi["s0"]).cuda().requires_grad_(True)
    o, sf = m.gated_delta_net_chunk(*(x[n] for n in GNAMES), initial_state=s0)
    (o.float() * synth.to_torch(d_o, "f32", "cuda")).sum().backward()
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gdn_fwd(*(gi[n] for n in GNAMES), gi["s0"])
    hz.check(dtype, hz.to_np(o), o_ref, hz.to_np(sf), s_ref, what=f"api gdn {dtype} o")
    ref = oracle.gdn_bwd(*(gi[n] for n in GNAMES), d_o, gi["s0"])
    for n in GNAMES:
        check_grad(dtype, hz.to_np(x[n].grad), ref[n], f"api gdn {dtype} d{n}")
    assert s0.grad.shape == (1, H, D, D)
    check_grad("f32", hz.to_np(s0.grad), ref["s0"], f"api gdn {dtype} ds0")


def test_one_token_forms():
    B, H, D = 3, 2, 64
    inp = synth.make(1, B=B, T=1, H=H, K=D, seed=8300, init=True, mask="none")
    x = {n: synth.to_torch(inp[n], "bf16", "cuda") for n in NAMES}
    s0 = torch.from_numpy(inp["s0"]).cuda()
    keep = s0.clone()
    o, nxt = m.rwkv7_op_rnn(*(x[n] for n in NAMES), initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == (B, 1, H, D)
    assert torch.equal(s0, keep), "the initial state must not be modified"
    o_ref, s_ref = oracle.step(*(inp[n][:, 0] for n in NAMES), inp["s0"])
    hz.check("bf16", hz.to_np(o)[:, 0], o_ref, hz.to_np(nxt), s_ref, what="api rwkv7_op_rnn")

    gi = synth.make_gdn(B, 1, H, D, seed=8301, init=True, n_state=1)
    g1 = {n: synth.to_torch(gi[n][:, 0], "bf16", "cuda") for n in GNAMES}
    gs0 = torch.from_numpy(gi["s0"]).cuda()
    o, nxt = m.gated_delta_net_recurrent_single_step(*(g1[n] for n in GNAMES), initial_state=gs0)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gdn_fwd(*(gi[n] for n in GNAMES), gi["s0"])
    hz.check("bf16", hz.to_np(o), o_ref[:, 0], hz.to_np(nxt), s_ref, what="api gdn single step")


def test_generalized_delta_rule_packed_autograd():
    """Packed sequences through autograd: the pool's gradient is the sum of
    the oracle's per-sequence initial-state gradients over the sequences
    mapped to each row (an entry outside the pool means a zero start)."""
    lengths, H, D = [20, 0, 37, 16], 2, 64
    TT = sum(lengths)
    inp = synth.make(1, B=1, T=TT, H=H, K=D, seed=8400, init=False, mask="bernoulli")
    rng = np.random.default_rng(8401)
    pool_np = (rng.standard_normal((3, H, D, D)) * 0.1).astype(np.float32)
    smap_np = np.array([2, 0, 2, 7], np.int32)
    d_o = synth.round_to(rng.standard_normal((1, TT, H, D)).astype(np.float32), "bf16")
    d_sf = (rng.standard_normal((len(lengths), H, D, D)) * 0.5).astype(np.float32)
    cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = {n: leaf(inp[n], "bf16") for n in NAMES}
    pool = torch.from_numpy(pool_np).cuda().requires_grad_(True)
    o, sf = m.generalized_delta_rule(*(x[n] for n in NAMES), initial_state=pool,
                                     mask=torch.from_numpy(inp["mask"]).cuda(),
                                     cu_seqlens=torch.from_numpy(cu_np).cuda(),
                                     state_map=torch.from_numpy(smap_np).cuda())
    loss = (o.float() * synth.to_torch(d_o, "f32", "cuda")).sum() + (sf * torch.from_numpy(d_sf).cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    ds0_pool = np.zeros_like(pool_np, dtype=np.float64)
    for n in range(len(lengths)):
        tb, te = int(cu_np[n]), int(cu_np[n + 1])
        row = int(smap_np[n])
        s0 = pool_np[row][None] if 0 <= row < 3 else None
        sl = {k: inp[k][:, tb:te] for k in NAMES}
        msk = inp["mask"][:, tb:te]
        o_ref, s_ref = oracle.fwd(*(sl[k] for k in NAMES), s0, msk)
        hz.check("bf16", hz.to_np(o)[:, tb:te], o_ref, hz.to_np(sf)[n:n + 1], s_ref, what=f"api packed seq{n} o")
        ref = oracle.bwd(*(sl[k] for k in NAMES), d_o[:, tb:te], s0, msk, d_sf[n][None])
        for k in NAMES:
            if te > tb:
                check_grad("bf16", hz.to_np(x[k].grad)[:, tb:te], ref[k], f"api packed seq{n} d{k}")
        if 0 <= row < 3:
            ds0_pool[row] += ref["s0"][0]
    check_grad("f32", hz.to_np(pool.grad), ds0_pool, "api packed pool ds0")


def test_gated_delta_net_packed_autograd_shared_row():
    """Packed Gated DeltaNet through autograd with one pool row shared by
    every sequence: its gradient is the sum of the oracle's per-sequence
    initial-state gradients."""
    lengths, H, D = [25, 0, 40], 2, 64
    TT = sum(lengths)
    gi = synth.make_gdn(1, TT, H, D, seed=8500)
    rng = np.random.default_rng(8501)
    pool_np = (rng.standard_normal((1, H, D, D)) * 0.1).astype(np.float32)
    d_o = synth.round_to(rng.standard_normal((1, TT, H, D)).astype(np.float32), "bf16")
    cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = {n: leaf(gi[n], "bf16") for n in GNAMES}
    pool = torch.from_numpy(pool_np).cuda().requires_grad_(True)
    o, sf = m.gated_delta_net(*(x[n] for n in GNAMES), initial_state=pool,
                              cu_seqlens=torch.from_numpy(cu_np).cuda())
    (o.float() * synth.to_torch(d_o, "f32", "cuda")).sum().backward()
    torch.cuda.synchronize()
    ds0 = np.zeros((1, H, D, D))
    for n in range(len(lengths)):
        tb, te = int(cu_np[n]), int(cu_np[n + 1])
        sl = {k: gi[k][:, tb:te] for k in GNAMES}
        o_ref, s_ref = oracle.gdn_fwd(*(sl[k] for k in GNAMES), pool_np)
        hz.check("bf16", hz.to_np(o)[:, tb:te], o_ref, hz.to_np(sf)[n:n + 1], s_ref, what=f"api gdn packed seq{n} o")
        ref = oracle.gdn_bwd(*(sl[k] for k in GNAMES), d_o[:, tb:te], pool_np)
        if te > tb:
            for k in GNAMES:
                check_grad("bf16", hz.to_np(x[k].grad)[:, tb:te], ref[k], f"api gdn packed seq{n} d{k}")
        ds0 += ref["s0"]
    check_grad("f32", hz.to_np(pool.grad), ds0, "api gdn packed shared ds0")

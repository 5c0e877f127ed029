"""GPU check of wkv7_bwd_noalloc, the allocation-free variant of wkv7_bwd
(its scratch is a fixed device array inside the library instead of a
caller workspace).  Through the C ABI it must give exactly what wkv7_bwd
gives on the same inputs -- the same kernels run on the same data -- on two
calls in a row, the second one smaller (the array keeps the first call's
contents), and both must match the fp64 oracle within the backward's
tolerance.
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
GRADS = NAMES + ("s0",)


def case(B, T, H, D, dtype, seed, shared=False):
    inp = synth.make(1, B=B, T=T, H=H, K=D, seed=seed, init=not shared, mask="bernoulli")
    for n in NAMES:
        inp[n] = synth.round_to(inp[n], dtype)
    rng = np.random.default_rng(seed + 1)
    if shared:
        inp["s0"] = (rng.standard_normal((1, H, D, D)) * 0.1).astype(np.float32)
    d_o = synth.round_to(rng.standard_normal((B, T, H, D)).astype(np.float32), dtype)
    d_sf = (rng.standard_normal((B, H, D, D)) * 0.5).astype(np.float32)
    dev = {n: synth.to_torch(inp[n], dtype, "cuda") for n in NAMES}
    dev["s0"] = torch.from_numpy(inp["s0"]).cuda()
    dev["mask"] = torch.from_numpy(inp["mask"]).cuda()
    dev["d_o"] = synth.to_torch(d_o, dtype, "cuda")
    dev["d_sf"] = torch.from_numpy(d_sf).cuda()
    return inp, d_o, d_sf, dev


def run_both(dev):
    args = [dev[n] for n in NAMES] + [dev["d_o"]]
    kw = dict(initial_state=dev["s0"], mask=dev["mask"], d_final_state=dev["d_sf"])
    g_ref = wkv7.bwd(*args, **kw)
    g_new = wkv7.bwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return g_ref, g_new


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 128)])
def test_noalloc_matches_bwd_two_calls_second_smaller(dtype, D):
    sizes = [(3, 300, 4), (2, 37, 2)]      # the second call is smaller
    for i, (B, T, H) in enumerate(sizes):
        shared = i == 1
        inp, d_o, d_sf, dev = case(B, T, H, D, dtype, seed=9100 + 10 * i + D, shared=shared)
        assert wkv7.bwd_workspace_bytes(B, T, H, D, D) <= wkv7.NOALLOC_SCRATCH_BYTES
        g_ref, g_new = run_both(dev)
        for n in GRADS:
            assert torch.equal(g_ref[n], g_new[n]), f"call {i}: d{n} differs from wkv7_bwd"
        s0 = np.repeat(inp["s0"], B, axis=0) if shared else inp["s0"]
        ref = oracle.bwd(*(inp[n] for n in NAMES), d_o, s0, inp["mask"], d_sf)
        if shared:
            ref["s0"] = ref["s0"].sum(axis=0, keepdims=True)
        for n in NAMES:
            check_grad(dtype, hz.to_np(g_new[n]), ref[n], f"noalloc call {i} D{D} d{n}")
        check_grad("f32", hz.to_np(g_new["s0"]), ref["s0"], f"noalloc call {i} D{D} ds0")


def test_noalloc_rejects_too_large_without_launch():
    """Sizes whose workspace exceeds the fixed array are refused on the host."""
    B, T, H, D = 1, 4096, 8, 64
    assert wkv7.bwd_workspace_bytes(B, T, H, D, D) > wkv7.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(wkv7.WKV7Error) as err:
        wkv7.bwd_noalloc(x, x, x, x, x, x, x)
    assert err.value.status == wkv7.ERR_TOO_LARGE

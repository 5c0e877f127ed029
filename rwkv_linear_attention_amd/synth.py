"""Seeded synthetic workloads for the WKV7 forward and decode step.

This module only draws inputs; it holds none of the operator's arithmetic,
and both the oracle side and the HIP side of every test consume what it
returns.  Shapes follow the RWKV-7 operator interface (rwkv-ops README,
section "rwkv7op 使用方法": r, w, k, a, b are [B,T,H,K], v is [B,T,H,V],
initial_state is [B,H,K,V], mask is [B,T]).

Value recipe (the same for every workload):
  r, v   ~ N(0, 1)
  k      ~ N(0, 1), then L2-normalised over K for every (b, t, h)
  w      = clip(-exp(N(-0.5, 0.5)), -5, -0.01)      (log-space decay, <= 0)
  kappa  ~ N(0, 1), L2-normalised over K;  iclr ~ U(0, 1) elementwise
  a      = -kappa,  b = kappa * iclr
  initial_state ~ N(0, 0.1) in fp32 when the workload has one
  mask   : Bernoulli(0.9) per token, or the last floor(T/10) tokens of every
           sequence set to 0 (trailing padding), or absent.
Draw order from numpy.random.default_rng(seed): r, v, k, w, kappa, iclr,
initial_state, mask.  Everything is drawn in fp32 and then rounded to the
I/O dtype (round-to-nearest-even for bf16); the fp32 state is not rounded.
"""
import numpy as np

WORKLOADS = [
    dict(index=0, name="fwd_f32_B1_T64_H1_d64", op="fwd", dtype="f32",
         B=1, T=64, H=1, K=64, init=False, mask=None),
    dict(index=1, name="fwd_bf16_B2_T1024_H4_d64_mask_s0", op="fwd", dtype="bf16",
         B=2, T=1024, H=4, K=64, init=True, mask="bernoulli"),
    dict(index=2, name="fwd_bf16_B8_T4096_H64_d64", op="fwd", dtype="bf16",
         B=8, T=4096, H=64, K=64, init=False, mask=None),
    dict(index=3, name="fwd_bf16_B16_T4096_H32_d128_pad_s0", op="fwd", dtype="bf16",
         B=16, T=4096, H=32, K=128, init=True, mask="trailing"),
    dict(index=4, name="step_bf16_B512_H40_d64_x256", op="step", dtype="bf16",
         B=512, T=256, H=40, K=64, init=True, mask=None),
]


def bf16_bits(x):
    """Round fp32 values to bf16 (nearest-even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x, dtype):
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return bf16_to_f32(bf16_bits(x))


def _unit(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True))
    return x / n


def make(workload, B=None, T=None, H=None, K=None, seed=None, init=None, mask=None):
    """Draw one workload.  Sizes, init and mask kind default to the workload's
    own; seed defaults to 1000 + workload index.  Returns a dict of numpy
    arrays: r, w, k, v, a, b (float32 holding values exactly representable in
    the I/O dtype), s0 (float32 or None), mask (uint8 or None), and dtype."""
    wl = WORKLOADS[workload] if isinstance(workload, int) else workload
    B = wl["B"] if B is None else B
    T = wl["T"] if T is None else T
    H = wl["H"] if H is None else H
    K = wl["K"] if K is None else K
    init = wl["init"] if init is None else init
    mask_kind = wl["mask"] if mask is None else (None if mask == "none" else mask)
    seed = 1000 + wl["index"] if seed is None else seed
    dt = wl["dtype"]
    rng = np.random.default_rng(seed)
    shp = (B, T, H, K)
    f = np.float32
    r = rng.standard_normal(shp, dtype=f)
    v = rng.standard_normal(shp, dtype=f)
    k = _unit(rng.standard_normal(shp, dtype=f))
    w = np.clip(-np.exp(rng.standard_normal(shp, dtype=f) * f(0.5) - f(0.5)), f(-5.0), f(-0.01))
    kappa = _unit(rng.standard_normal(shp, dtype=f))
    iclr = rng.random(shp, dtype=f)
    a = -kappa
    b = kappa * iclr
    del kappa, iclr
    s0 = (rng.standard_normal((B, H, K, K), dtype=f) * f(0.1)) if init else None
    if mask_kind is None:
        m = None
    elif mask_kind == "bernoulli":
        m = (rng.random((B, T)) < 0.9).astype(np.uint8)
    elif mask_kind == "trailing":
        m = np.ones((B, T), np.uint8)
        n = T // 10
        if n:
            m[:, T - n:] = 0
    else:
        raise ValueError(mask_kind)
    out = dict(dtype=dt, s0=s0, mask=m)
    for name, x in (("r", r), ("w", w), ("k", k), ("v", v), ("a", a), ("b", b)):
        out[name] = round_to(x, dt)
    return out


def make_gdn(B, T, H, K, seed, dtype="bf16", init=False, n_state=None):
    """Draw one Gated DeltaNet workload (rwkv-ops README, section
    "gdn_recurrent 使用方法": q, k [B,T,H,K], v [B,T,H,V], g and beta [B,T,H],
    initial_state [B or 1,H,K,V]).

    Value recipe: q, k, v ~ N(0, 1) (raw: the operator normalises q and k);
    g = clip(-exp(N(-1.5, 0.75)), -8, -1e-3) (log-space gate, <= 0);
    beta = sigmoid(N(0, 1)) in (0, 1); initial_state ~ N(0, 0.1) fp32 with
    n_state rows (B by default) when init is set.  Draw order from
    numpy.random.default_rng(seed): q, k, v, g, beta, initial_state; all
    rounded to the I/O dtype except the fp32 state."""
    rng = np.random.default_rng(seed)
    f = np.float32
    shp = (B, T, H, K)
    q = rng.standard_normal(shp, dtype=f)
    k = rng.standard_normal(shp, dtype=f)
    v = rng.standard_normal(shp, dtype=f)
    g = np.clip(-np.exp(rng.standard_normal((B, T, H), dtype=f) * f(0.75) - f(1.5)), f(-8.0), f(-1e-3))
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H), dtype=f)))).astype(f)
    ns = B if n_state is None else n_state
    s0 = (rng.standard_normal((ns, H, K, K), dtype=f) * f(0.1)) if init else None
    out = dict(dtype=dtype, s0=s0)
    for name, x in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        out[name] = round_to(x, dtype)
    return out


def to_torch(x, dtype, device):
    """Move an array holding I/O-dtype values to a torch tensor of that dtype."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    bits = bf16_bits(x)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)


def make_device(workload, device, seed, B=None, T=None, H=None, K=None, step_major=False):
    """Draw a workload with the same value recipe as make(), on the device
    with torch's seeded generator (a different random stream from make()'s
    numpy one, and much faster at full size).  Returns a dict of device
    tensors in the I/O dtype -- r, w, k, v, a, b as [B,T,H,K], or [T,B,H,K]
    with step_major (so that one decode step's inputs are contiguous) -- and
    s0 (fp32 or None), mask (uint8 [B,T] or None), dtype."""
    import torch
    wl = WORKLOADS[workload] if isinstance(workload, int) else workload
    B = wl["B"] if B is None else B
    T = wl["T"] if T is None else T
    H = wl["H"] if H is None else H
    K = wl["K"] if K is None else K
    dt = torch.float32 if wl["dtype"] == "f32" else torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shp = (T, B, H, K) if step_major else (B, T, H, K)
    randn = lambda: torch.randn(shp, generator=g, device=device, dtype=torch.float32)
    unit = lambda x: x / torch.sqrt(torch.sum(x * x, dim=-1, keepdim=True))
    out = {"dtype": wl["dtype"]}
    out["r"] = randn().to(dt)
    out["v"] = randn().to(dt)
    out["k"] = unit(randn()).to(dt)
    out["w"] = torch.clamp(-torch.exp(randn() * 0.5 - 0.5), -5.0, -0.01).to(dt)
    kappa = unit(randn())
    out["a"] = (-kappa).to(dt)
    out["b"] = (kappa * torch.rand(shp, generator=g, device=device, dtype=torch.float32)).to(dt)
    del kappa
    out["s0"] = torch.randn((B, H, K, K), generator=g, device=device, dtype=torch.float32) * 0.1 \
        if wl["init"] else None
    if wl["mask"] == "trailing":
        m = torch.ones((B, T), dtype=torch.uint8, device=device)
        if T // 10:
            m[:, T - T // 10:] = 0
        out["mask"] = m
    elif wl["mask"] == "bernoulli":
        out["mask"] = (torch.rand((B, T), generator=g, device=device) < 0.9).to(torch.uint8)
    else:
        out["mask"] = None
    return out

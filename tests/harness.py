"""Shared helpers for the GPU parity tests: seeded inputs, both sides, and
the comparison rules.

Tolerances (from the operator's accuracy target):
  fp32 I/O: max |o - o_ref| <= 1e-4 and max |S - S_ref| <= 1e-4.
  bf16 I/O: max_i |o_i - o_ref,i| <= 0.02 * RMS(o_ref) + 2^-8 * |o_ref,i|
            (the RMS-relative bound plus one bf16 half-ulp, since rounding
            an exact output to bf16 alone already costs up to 2^-9 |o|), and
            max |S - S_ref| <= 0.02 * RMS(S_ref) for the fp32 final state.
"""
import json
import os

import numpy as np

import oracle
from rwkv_linear_attention_amd import synth

ARRAYS = ("r", "w", "k", "v", "a", "b")


def to_dev(inp, device="cuda"):
    import torch
    dt = inp["dtype"]
    out = {n: synth.to_torch(inp[n], dt, device) for n in ARRAYS}
    out["s0"] = None if inp["s0"] is None else torch.from_numpy(inp["s0"]).to(device)
    out["mask"] = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).to(device)
    return out


def gpu_fwd(dev, algo=0, output_final_state=True):
    from rwkv_linear_attention_amd import wkv7
    return wkv7.fwd(dev["r"], dev["w"], dev["k"], dev["v"], dev["a"], dev["b"],
                    initial_state=dev["s0"], mask=dev["mask"],
                    output_final_state=output_final_state, algo=algo)


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def oracle_fwd(inp, bh=None):
    """Oracle on all (b, h) or on the listed (b, h) pairs (returns lists)."""
    if bh is None:
        return oracle.fwd(inp["r"], inp["w"], inp["k"], inp["v"], inp["a"], inp["b"],
                          inp["s0"], inp["mask"])
    outs = []
    for (bb, h) in bh:
        sl = lambda x: x[bb:bb + 1, :, h:h + 1]
        s0 = None if inp["s0"] is None else inp["s0"][bb:bb + 1, h:h + 1]
        m = None if inp["mask"] is None else inp["mask"][bb:bb + 1]
        o, s = oracle.fwd(sl(inp["r"]), sl(inp["w"]), sl(inp["k"]), sl(inp["v"]),
                          sl(inp["a"]), sl(inp["b"]), s0, m)
        outs.append((o[0, :, 0], s[0, 0]))
    return outs


def _log(what, ratio):
    """Record the worst error / tolerance ratio when WKV7_PARITY_LOG names a file."""
    path = os.environ.get("WKV7_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": what, "ratio": round(float(ratio), 4)}) + "\n")


def check(dtype, o, o_ref, s=None, s_ref=None, what="", scale=1.0):
    """scale=2 compares two GPU results, each within the bound of the exact
    value (triangle inequality)."""
    o = np.asarray(o, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    if dtype == "f32":
        assert err.max(initial=0.0) <= 1e-4 * scale, f"{what}: max |do| = {err.max()}"
        if s is not None:
            es = np.abs(np.asarray(s) - s_ref).max(initial=0.0)
            assert es <= 1e-4 * scale, f"{what}: max |dS| = {es}"
        return err.max(initial=0.0)
    rms = float(np.sqrt(np.mean(o_ref ** 2))) if o_ref.size else 0.0
    allow = scale * (0.02 * rms + 2.0 ** -8 * np.abs(o_ref))
    ratio = float(np.max(err / np.maximum(allow, 1e-30))) if o.size else 0.0
    _log(what, ratio)
    assert ratio <= 1.0, f"{what}: worst error {ratio:.3f} x tolerance (RMS {rms:.4g})"
    if s is not None:
        s = np.asarray(s, np.float64)
        srms = float(np.sqrt(np.mean(np.asarray(s_ref) ** 2)))
        es = float(np.abs(s - s_ref).max(initial=0.0))
        assert es <= scale * 0.02 * srms or es == 0.0, f"{what}: max |dS| = {es:.3g} vs 0.02*RMS = {0.02 * srms:.3g}"
    return ratio


def check_grad(dtype, got, ref, what, floor=0.0):
    """Tolerance relative to the reference tensor's RMS.

    floor: the scale for a gradient tensor that vanishes identically, such as
    dw of a one-token sequence without an initial state (w only scales a zero
    state there).  Such a tensor has no scale of its own, and the chunk form
    builds it from O(1) terms that cancel exactly, so its fp32 rounding
    follows the size of those terms (the call's other input gradients).  The
    floor applies only when the oracle tensor is identically zero, or below
    1e-6 of the floor (fp64 round-off of an exact zero); every other tensor is
    held to its own RMS."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    if floor > 0.0 and rms <= 1e-6 * floor:
        rms = floor
    if dtype == "bf16":
        allow = 0.02 * rms + 2.0 ** -8 * np.abs(ref)
    else:
        allow = 1e-4 * rms + 1e-5 * np.abs(ref)
    err = np.abs(got - ref)
    ratio = float(np.max(err / np.maximum(allow, 1e-30))) if got.size else 0.0
    _log(what, ratio)
    assert ratio <= 1.0 or np.all(err == 0), f"{what}: worst error {ratio:.3f} x tolerance (RMS {rms:.3g})"


def check_sequences(dtype, o, o_ref, s, s_ref, what):
    """Element-by-element check of every (b, h) sequence of a full-size call,
    each against its own output RMS: o, o_ref [B,T,H,V]; s, s_ref [B,H,K,V]
    (torch tensors on the device or numpy arrays).  The rules are those of
    check(); batches are converted one at a time to bound host memory.
    Returns the worst (output, state) error / tolerance ratios."""
    B, H = o_ref.shape[0], o_ref.shape[2]
    worst_o = worst_s = 0.0
    for bb in range(B):
        ob = to_np(o[bb]) if not isinstance(o, np.ndarray) else np.asarray(o[bb], np.float64)
        rb = np.asarray(o_ref[bb], np.float64)                      # [T, H, V]
        sb = to_np(s[bb]) if not isinstance(s, np.ndarray) else np.asarray(s[bb], np.float64)
        srb = np.asarray(s_ref[bb], np.float64)                     # [H, K, V]
        assert np.all(np.isfinite(ob)), f"{what} b={bb}: non-finite output"
        err = np.abs(ob - rb)
        serr = np.abs(sb - srb).reshape(H, -1).max(axis=1)
        if dtype == "f32":
            ro = err.reshape(-1, H, err.shape[-1]).max(axis=(0, 2)) / 1e-4
            rs = serr / 1e-4
        else:
            rms = np.sqrt(np.mean(rb ** 2, axis=(0, 2)))             # per head
            allow = 0.02 * rms[None, :, None] + 2.0 ** -8 * np.abs(rb)
            ro = (err / np.maximum(allow, 1e-30)).max(axis=(0, 2)) if rb.shape[0] else np.zeros(H)
            srms = np.sqrt(np.mean(srb.reshape(H, -1) ** 2, axis=1))
            rs = np.where(serr == 0.0, 0.0, serr / np.maximum(0.02 * srms, 1e-30))
        ho, hs = int(np.argmax(ro)), int(np.argmax(rs))
        assert ro[ho] <= 1.0, f"{what} (b={bb}, h={ho}): worst output error {ro[ho]:.3f} x tolerance"
        assert rs[hs] <= 1.0, f"{what} (b={bb}, h={hs}): worst state error {rs[hs]:.3f} x tolerance"
        worst_o, worst_s = max(worst_o, float(ro.max())), max(worst_s, float(rs.max()))
    _log(what + " o", worst_o)
    _log(what + " final state", worst_s)
    return worst_o, worst_s

"""Benchmark of the WKV7 forward (bf16 I/O, fp32 state) on one MI355X.

A step is one wkv7_fwd call over the whole B=8, T=4096, H=64, K=V=64 batch
(the chunked kernel, selected by ALGO_AUTO), inputs resident in HBM.  Prints
one JSON line with Mtokens/s, the dominant kernel's HBM roofline fraction
(algorithmic bytes / measured launch time vs 8 TB/s), and the fp64 CPU oracle
timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# MI355X published fp32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2 (packed fp32) x 2 flops (FMA)
# x 2.4 GHz.  Code built without packed fp32 instructions issues at most half of it.
FP32_VECTOR_PEAK_TFLOPS = 157.3
PROFILE_NOTE = os.path.join(ROOT, "profiles", "wkv7_chunked_B8_T4096_H64_d64.md")
PROFILE_NOTE_D128 = os.path.join(ROOT, "profiles", "wkv7_chunked_B16_T4096_H32_d128.md")
PROFILE_NOTE_STEP = os.path.join(ROOT, "profiles", "wkv7_step_B512_H40_d64.md")
CSRC = os.path.join(ROOT, "rwkv_linear_attention_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("wkv7_chunked.hip", "wkv7_common.hpp")]
STEP_SOURCES = [os.path.join(CSRC, f) for f in ("wkv7_step.hip", "wkv7_common.hpp")]


def kernel_sha(sources=None):
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(B, T, H, D, dtype_bytes, has_s0, has_final, has_mask):
    """Inputs once (r, w, k, v, a, b), o once, states once, mask 1 B/token."""
    tok = B * T * H * D * dtype_bytes
    st = B * H * D * D * 4
    return 6 * tok + tok + (st if has_s0 else 0) + (st if has_final else 0) + (B * T if has_mask else 0)


def measured_traffic(sha, note=PROFILE_NOTE):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, each scaled by what the
    counter reads for a plain copy of known size), if it was taken on this
    exact kernel source; otherwise None."""
    if not os.path.exists(note):
        return None
    txt = open(note).read()
    m = re.search(r"traffic: source_sha=(\w+) fetch_kib=([\d.]+) fetch_scale=([\d.]+) "
                  r"write_kib=([\d.]+) write_scale=([\d.]+)", txt)
    if not m or m.group(1) != sha:
        return None
    fk, fs, wk, ws = (float(m.group(i)) for i in range(2, 6))
    return round((fk * fs + wk * ws) * 1024.0)


def cpu_baseline(inp, H, T, budget_s=12.0, max_threads=16):
    """Time the fp64 oracle on whole (b, h) sequences of the same workload
    until about budget_s seconds of work; report full-workload tokens/s."""
    import numpy as np
    import oracle
    threads = min(max_threads, len(os.sched_getaffinity(0)))
    oracle.set_threads(threads)
    B = inp["r"].shape[0]
    pairs = [(bb, h) for h in range(H) for bb in range(B)]
    done, t_used, batch = 0, 0.0, threads
    while t_used < budget_s:
        lo = done % len(pairs)
        sel = pairs[lo:lo + batch]
        # gather the selected sequences as a [n, T, 1, D] batch
        g = lambda n: np.stack([inp[n][bb, :, h] for bb, h in sel])[:, :, None, :]
        args = [g(n) for n in ("r", "w", "k", "v", "a", "b")]
        t0 = time.perf_counter()
        oracle.fwd(*args)
        t_used += time.perf_counter() - t0
        done += len(sel)
        batch = min(batch * 2, 4 * threads * 8)
    seq_tokens = done * T                    # single-head tokens processed
    full_tokens = seq_tokens / H             # = tokens of the workload (all heads)
    # one thread on a few whole sequences, extrapolated to the workload
    oracle.set_threads(1)
    n1 = 8
    sel = pairs[:n1]
    g = lambda n: np.stack([inp[n][bb, :, h] for bb, h in sel])[:, :, None, :]
    args = [g(n) for n in ("r", "w", "k", "v", "a", "b")]
    t0 = time.perf_counter()
    oracle.fwd(*args)
    t1 = time.perf_counter() - t0
    oracle.set_threads(threads)
    return {"value": full_tokens / t_used / 1e6, "unit": "Mtokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} (b,h) sequences of T={T} ({done / len(pairs):.2f} passes over the "
                      f"{len(pairs)} sequences of the workload; fp64 C, OpenMP), {t_used:.1f} s",
            "single_thread": {"value": round(n1 * T / H / t1 / 1e6, 6), "unit": "Mtokens/s",
                              "extrapolated_workload_s": round(t1 / n1 * len(pairs), 1),
                              "sample": f"{n1} (b,h) sequences of T={T} on one thread, {t1:.2f} s, "
                                        f"extrapolated to the {len(pairs)} sequences of the workload"}}


def oracle_sample_rate(call, B, H, T, budget_s=4.0, max_threads=16):
    """Time call(pairs) -- the fp64 oracle on a list of (b, h) sequences --
    on growing batches until about budget_s seconds of work; report the rate
    scaled to the whole workload (tokens of all heads) in Mtokens/s."""
    import oracle
    threads = min(max_threads, len(os.sched_getaffinity(0)))
    oracle.set_threads(threads)
    pairs = [(bb, h) for h in range(H) for bb in range(B)]
    done, t_used, batch = 0, 0.0, threads
    while t_used < budget_s and done < len(pairs):
        sel = pairs[done:done + batch]
        t0 = time.perf_counter()
        call(sel)
        t_used += time.perf_counter() - t0
        done += len(sel)
        batch = min(batch * 2, 8 * threads)
    return {"value": round(done * T / H / t_used / 1e6, 5), "unit": "Mtokens/s", "cores": threads,
            "kind": "oracle", "sample": f"{done} (b,h) sequences of T={T} (fp64 C, OpenMP), {t_used:.1f} s"}


SETTLE_MS = 100.0


def copy_context(nbytes=1 << 30, reps=20):
    """Achievable-bandwidth context: a plain device-to-device copy of 1 GiB
    (torch's copy kernel; 2 GiB moved per copy), timed after the clock
    settle like the workloads."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    settle(lambda: dst.copy_(src))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "device-to-device copy of 1 GiB (read + write)", "ms": round(ms, 4),
            "GB_per_s": round(2 * nbytes / ms / 1e6, 1), "frac_of_8TBps": round(2 * nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}


def settle(fn, ms=SETTLE_MS):
    """Run fn (untimed) until `ms` of wall time have passed; returns the call
    count.  From idle the GPU raises its clocks over the first ~25 ms of
    sustained work (the B8 T4096 d64 forward measured 0.60 ms per launch in
    its first 10 launches, 0.40 ms from about the 60th on), so a few warmup
    steps alone would time the ramp rather than the kernel."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        n += 5
    return n


def time_steps(step, steps, warmup):
    """Clock settle, W untimed steps, then K timed steps with a HIP event
    pair around each launch (torch's current stream, where the library
    launches) and one around all of them.  Returns (ms per step over the
    whole timed region, mean launch duration in ms, settle step count)."""
    import torch
    n_settle = settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps, n_settle


def _host_sequences(x, pairs, names):
    """The listed (b, h) sequences of [B,T,H,K] device tensors as float64
    host arrays [n, T, 1, K] (inputs for the oracle)."""
    import numpy as np
    import torch
    idx_b = torch.tensor([p[0] for p in pairs], device=x[names[0]].device)
    idx_h = torch.tensor([p[1] for p in pairs], device=x[names[0]].device)
    return {n: x[n][idx_b, :, idx_h].float().cpu().numpy().astype(np.float64)[:, :, None, :] for n in names}


def d128_entry(steps, warmup, cpu=True):
    """Workload 3: bf16 B16 T4096 H32 K=V=128 forward with a random initial
    state and a trailing-padding mask (10 % of each sequence), final state
    written; chunked kernel under AUTO.  Inputs drawn on the device (same
    recipe as the parity tests, torch's generator)."""
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    wl = synth.WORKLOADS[3]
    B, T, H, D = wl["B"], wl["T"], wl["H"], wl["K"]
    print(f"[bench] generating workload {wl['name']} on the device", file=sys.stderr, flush=True)
    x = synth.make_device(3, "cuda", seed=2003)
    names = ("r", "w", "k", "v", "a", "b")
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    path = wkv7.fwd_path(torch.bfloat16, B, T, H, D, D)
    assert path == wkv7.ALGO_CHUNKED
    step = lambda: wkv7.fwd(*(x[n] for n in names), initial_state=x["s0"], mask=x["mask"], out=o, final_state=sf)
    ms_step, launch_ms, _ = time_steps(step, steps, warmup)
    nbytes = algorithmic_bytes(B, T, H, D, 2, True, True, True)
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    sha = kernel_sha()
    res = {"value": round(B * T / (ms_step * 1e-3) / 1e6, 3), "unit": "Mtokens/s", "steps": steps,
           "ms_per_step": round(ms_step, 5), "dtype": "bf16", "data": "synthetic (device generator, seed 2003)",
           "config": {"workload": wl["name"], "B": B, "T": T, "H": H, "K": D, "V": D, "C": H * D,
                      "initial_state": "random N(0, 0.1)", "mask": "last 409 tokens of each sequence 0",
                      "final_state": True, "kernel": "chunked"},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(sha, PROFILE_NOTE_D128), "algorithmic_bytes": nbytes,
                        "kernel_ms": round(launch_ms, 5), "kernel_sha": sha}}
    if cpu:
        import oracle

        def call(sel):
            h = _host_sequences(x, sel, names)
            s0 = x["s0"][[p[0] for p in sel], [p[1] for p in sel]].cpu().numpy()[:, None]
            m = x["mask"][[p[0] for p in sel]].cpu().numpy()
            oracle.fwd(*(h[n] for n in names), s0, m)
        print("[bench] timing the CPU oracle (head size 128) on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = oracle_sample_rate(call, B, H, T, budget_s=6.0)
    del x, o, sf
    torch.cuda.empty_cache()
    return {wl["name"]: res}


def decode_entry(reps, cpu=True):
    """Workload 4: 256 consecutive wkv7_step calls (bf16 inputs, fp32 state
    updated in place) on B512 H40 K=V=64 from a random initial state, fresh
    inputs every step (256 distinct steps drawn on the device, step-major so
    each step's inputs are contiguous).  The state is reset from a pristine
    copy before each repetition, outside the timed region."""
    import numpy as np
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    wl = synth.WORKLOADS[4]
    B, NSTEP, H, D = wl["B"], wl["T"], wl["H"], wl["K"]
    print(f"[bench] generating workload {wl['name']} on the device", file=sys.stderr, flush=True)
    x = synth.make_device(4, "cuda", seed=2004, step_major=True)      # [256, B, H, D]
    names = ("r", "w", "k", "v", "a", "b")
    state0 = x["s0"]
    state = state0.clone()
    obuf = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")

    def run():
        state.copy_(state0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(NSTEP):
            wkv7.step(*(x[n][t] for n in names), state, out=obuf)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    settle(lambda: wkv7.step(*(x[n][0] for n in names), state, out=obuf))
    run()
    ms_total = sum(run() for _ in range(reps)) / reps
    launch_ms = ms_total / NSTEP
    step_bytes = 2 * B * H * D * D * 4 + 6 * B * H * D * 2 + B * H * D * 2
    achieved = step_bytes / (launch_ms * 1e-3) / 1e9
    sha = kernel_sha(STEP_SOURCES)
    res = {"value": round(B * NSTEP / (ms_total * 1e-3) / 1e6, 3), "unit": "Mtokens/s", "steps": reps,
           "ms_per_step": round(ms_total, 4), "us_per_decode_step": round(launch_ms * 1e3, 2), "dtype": "bf16",
           "data": "synthetic (device generator, seed 2004)",
           "config": {"workload": wl["name"], "B": B, "H": H, "K": D, "V": D, "C": H * D,
                      "decode_steps": NSTEP, "initial_state": "random N(0, 0.1)", "kernel": "step"},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(sha, PROFILE_NOTE_STEP), "algorithmic_bytes": step_bytes,
                        "kernel_ms": round(launch_ms, 5), "kernel_sha": sha,
                        "note": "per step launch: state read and written, inputs and o once"}}
    if cpu:
        import oracle
        threads = min(16, len(os.sched_getaffinity(0)))
        oracle.set_threads(threads)
        print("[bench] timing the CPU oracle (decode) on whole steps", file=sys.stderr, flush=True)
        S = state0.cpu().numpy().astype(np.float64)
        n, t_used = 0, 0.0
        while t_used < 4.0 and n < NSTEP:
            h = {m: x[m][n].float().cpu().numpy() for m in names}
            t0 = time.perf_counter()
            _, S = oracle.step(*(h[m] for m in names), S)
            t_used += time.perf_counter() - t0
            n += 1
        res["cpu_baseline"] = {"value": round(B * n / t_used / 1e6, 6), "unit": "Mtokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the first {n} of the 256 decode steps, all {B * H} sequences each "
                                         f"(fp64 C, OpenMP), {t_used:.1f} s"}
    del x, state, state0, obuf
    torch.cuda.empty_cache()
    return {wl["name"]: res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--all", action="store_true",
                    help="also time the head-size-128 workload, a packed variable-length batch, Gated "
                         "DeltaNet, the backward and the 256-step decode")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--dispatch-sweep", action="store_true",
                    help="time the recurrent and chunked kernels over T and B*H (bf16) and print "
                         "one JSON line per shape; used to set the AUTO thresholds")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the operator is independent per (batch, head), "
              "so N GPUs run N disjoint batch/head shards with no communication; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rwkv_linear_attention_amd import synth, wkv7

    if args.dispatch_sweep:
        dispatch_sweep()
        return

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)
        return

    wl = synth.WORKLOADS[2]
    B, T, H, D = wl["B"], wl["T"], wl["H"], wl["K"]
    print(f"[bench] generating workload {wl['name']}", file=sys.stderr, flush=True)
    inp = synth.make(2)
    dev = {n: synth.to_torch(inp[n], "bf16", "cuda") for n in ("r", "w", "k", "v", "a", "b")}
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    path = wkv7.fwd_path(torch.bfloat16, B, T, H, D, D)
    assert path == wkv7.ALGO_CHUNKED

    def step():
        wkv7.fwd(dev["r"], dev["w"], dev["k"], dev["v"], dev["a"], dev["b"],
                 out=o, final_state=sf)

    print(f"[bench] clock settle, {args.warmup} warmup steps, {args.steps} timed steps", file=sys.stderr, flush=True)
    ms_per_step, launch_ms, n_settle = time_steps(step, args.steps, args.warmup)

    alg_bytes = algorithmic_bytes(B, T, H, D, 2, False, True, False)
    achieved = alg_bytes / (launch_ms * 1e-3) / 1e9
    sha = kernel_sha()
    traffic = measured_traffic(sha)
    tokens = B * T
    result = {
        "metric": "WKV7 fwd Mtokens/s + % HBM roofline, B8 T4096 C4096 hd64 bf16",
        "value": round(tokens / (ms_per_step * 1e-3) / 1e6, 3),
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"ms": SETTLE_MS, "steps": n_settle},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["name"], "B": B, "T": T, "H": H, "K": D, "V": D, "C": H * D,
                   "initial_state": None, "mask": None, "final_state": True, "kernel": "chunked"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": alg_bytes,
                     "kernel_ms": round(launch_ms, 5), "kernel_sha": sha},
    }
    result["copy_context"] = copy_context()
    if not args.no_cpu:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, H, T)
    del dev, o, sf, inp
    torch.cuda.empty_cache()
    # the two other full-size workloads, each with its own roofline and CPU baseline
    result["others"] = d128_entry(args.steps, args.warmup, not args.no_cpu)
    result["others"].update(decode_entry(max(3, args.steps // 10), not args.no_cpu))
    if args.all:
        result["more"] = other_workloads(args.steps, args.warmup, not args.no_cpu)
    print(json.dumps(result), flush=True)


def dispatch_sweep(reps=10, dtypes=("bf16", "f32")):
    """Recurrent vs chunked launch time (no state in, final state out) for
    both I/O types, head sizes 64 and 128, B*H sequences in {1, 8, 64, 512}
    (as B = 1, H = B*H), T from 1 to 2048.  One JSON line per shape."""
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    for dt in dtypes:
      tdt = torch.bfloat16 if dt == "bf16" else torch.float32
      for D in (64, 128):
        for BH in (1, 8, 64, 512):
            for T in (1, 2, 4, 8, 16, 32, 48, 64, 96, 128, 256, 512, 1024, 2048):
                inp = synth.make(dict(synth.WORKLOADS[2], dtype=dt), B=1, T=T, H=BH, K=D, seed=7)
                dev = {n: synth.to_torch(inp[n], dt, "cuda") for n in ("r", "w", "k", "v", "a", "b")}
                o = torch.empty((1, T, BH, D), dtype=tdt, device="cuda")
                sf = torch.empty((1, BH, D, D), dtype=torch.float32, device="cuda")
                res = {"dtype": dt, "D": D, "BH": BH, "T": T}
                for name, algo in (("recurrent_us", wkv7.ALGO_RECURRENT), ("chunked_us", wkv7.ALGO_CHUNKED)):
                    ms = _time_launches(lambda i: wkv7.fwd(*(dev[n] for n in ("r", "w", "k", "v", "a", "b")),
                                                           out=o, final_state=sf, algo=algo), reps, 2)
                    res[name] = round(ms * 1e3, 2)
                res["auto"] = "chunked" if wkv7.fwd_path(tdt, 1, T, BH, D, D) == wkv7.ALGO_CHUNKED else "recurrent"
                print(json.dumps(res), flush=True)
                del dev, o, sf, inp


def varlen_lengths(total, n, seed):
    """Seeded mix of n sequence lengths in [16, 4096) summing to total."""
    import numpy as np
    rng = np.random.default_rng(seed)
    x = rng.lognormal(mean=0.0, sigma=0.8, size=n)
    lens = np.maximum(16, np.floor(x / x.sum() * total)).astype(np.int64)
    lens = np.minimum(lens, 4095)
    lens[np.argmax(lens)] += total - int(lens.sum())
    return lens


def varlen_workload(steps, warmup):
    """Packed variable-length forward: the 32768 tokens x 64 heads (d64) of
    the B8 T4096 workload as 32 sequences of mixed lengths, each starting from
    one of 8 pooled initial states (state_map), final states written; then
    the backward of the same packed forward."""
    import numpy as np
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    H, D, N, TT = 64, 64, 32, 8 * 4096
    lens = varlen_lengths(TT, N, seed=1207)
    print(f"[bench] generating packed workload (N={N}, lengths {int(lens.min())}..{int(lens.max())})",
          file=sys.stderr, flush=True)
    inp = synth.make(2, B=1, T=TT, H=H, K=D, seed=1207)
    dev = {n: synth.to_torch(inp[n][0], "bf16", "cuda") for n in ("r", "w", "k", "v", "a", "b")}
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    rng = np.random.default_rng(1208)
    pool = torch.from_numpy((rng.standard_normal((8, H, D, D)) * 0.1).astype(np.float32)).cuda()
    smap = torch.from_numpy(rng.integers(0, 8, size=N).astype(np.int32)).cuda()
    o = torch.empty((TT, H, D), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    ms = _time_launches(lambda i: wkv7.fwd_varlen(*(dev[n] for n in ("r", "w", "k", "v", "a", "b")), cu,
                                                  initial_state=pool, state_map=smap, out=o, final_state=sf),
                        steps, warmup)
    # inputs and o once, one mapped initial state read and one final state written per sequence
    nbytes = 7 * TT * H * D * 2 + 2 * N * H * D * D * 4
    name = f"fwd_varlen_bf16_N{N}_T{TT}_H{H}_d{D}_statemap8"
    res = {name: {"ms": round(ms, 5), "Mtokens_per_s": round(TT / ms / 1e3, 3),
                  "GB_per_s": round(nbytes / ms / 1e6, 1),
                  "frac_of_8TBps": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
                  "lengths": [int(x) for x in lens], "kernel": "chunked d64 (packed)"}}
    del o, sf
    # a skewed packed batch under AUTO: 299 one-token sequences and one of
    # 4096 tokens (mean length 14.6), beside the single 4096-token sequence
    # alone on the chunked kernel
    sk_lens = [1] * 299 + [4096]
    STT = sum(sk_lens)
    sk = synth.make(2, B=1, T=STT, H=H, K=D, seed=1209)
    sdev = {n: synth.to_torch(sk[n][0], "bf16", "cuda") for n in ("r", "w", "k", "v", "a", "b")}
    scu = torch.from_numpy(np.concatenate([[0], np.cumsum(sk_lens)]).astype(np.int32)).cuda()
    so = torch.empty((STT, H, D), dtype=torch.bfloat16, device="cuda")
    ssf = torch.empty((len(sk_lens), H, D, D), dtype=torch.float32, device="cuda")
    ms_sk = _time_launches(lambda i: wkv7.fwd_varlen(*(sdev[n] for n in ("r", "w", "k", "v", "a", "b")), scu,
                                                     out=so, final_state=ssf), steps, warmup)
    one = {n: sdev[n][299:].unsqueeze(0) for n in sdev}
    o1 = torch.empty((1, 4096, H, D), dtype=torch.bfloat16, device="cuda")
    s1 = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    ms_one = _time_launches(lambda i: wkv7.fwd(*(one[n] for n in ("r", "w", "k", "v", "a", "b")), out=o1,
                                               final_state=s1, algo=wkv7.ALGO_CHUNKED), steps, warmup)
    ms_rec = _time_launches(lambda i: wkv7.fwd_varlen(*(sdev[n] for n in ("r", "w", "k", "v", "a", "b")), scu,
                                                      out=so, final_state=ssf, algo=wkv7.ALGO_RECURRENT),
                            max(3, steps // 5), 1)
    res[f"fwd_varlen_bf16_skewed_299x1_1x4096_H{H}_d{D}"] = {
        "ms_auto": round(ms_sk, 5), "ms_forced_recurrent": round(ms_rec, 5),
        "ms_long_sequence_alone_chunked": round(ms_one, 5),
        "note": "AUTO takes the chunked kernel for packed bf16; the long sequence sets the time"}
    del sk, sdev, so, ssf, one, o1, s1
    # the backward of the same packed forward (seeded N(0, 1) output gradient)
    d_o = synth.to_torch(synth.round_to(rng.standard_normal((TT, H, D), dtype=np.float32), "bf16"), "bf16", "cuda")
    ws = torch.empty(wkv7.bwd_varlen_workspace_bytes(N, TT, H, D, D), dtype=torch.uint8, device="cuda")
    gbuf = {n: torch.empty_like(dev[n]) for n in ("r", "w", "k", "v", "a", "b")}
    gbuf["s0"] = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    ms = _time_launches(lambda i: wkv7.bwd_varlen(*(dev[n] for n in ("r", "w", "k", "v", "a", "b")), cu, d_o,
                                                  initial_state=pool, state_map=smap, workspace=ws, out=gbuf),
                        max(3, steps // 4), max(1, warmup // 4))
    tok = TT * H * D * 2
    nbytes = 7 * tok + 6 * tok + 2 * N * H * D * D * 4
    # the packed chunks: sum of ceil(len / 16), the flop count of bwd_flops
    nck = int(sum((int(x) + 15) // 16 for x in lens))
    fl = 2 * nck * H * (13 * 16 * D * D + 30 * 16 * 16 * D)
    tf = fl / (ms * 1e-3) / 1e12
    res[f"bwd_varlen_bf16_N{N}_T{TT}_H{H}_d{D}_statemap8"] = {
        "ms": round(ms, 4), "Mtokens_per_s": round(TT / ms / 1e3, 3), "GB_per_s": round(nbytes / ms / 1e6, 1),
        "frac_of_8TBps": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
        "roofline": {"bound": "mfma", "unit": "TFLOP/s", "peak": FP32_MFMA_PEAK_TFLOPS, "achieved": round(tf, 2),
                     "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4), "flops": fl, "dtype": "f32"},
        "workspace_bytes": ws.numel(), "kernel": "recurrences + per-chunk gradients, d64 (packed)"}
    return res


def gdn_workload(steps, warmup, cpu=True):
    """Gated DeltaNet forward on the chunked kernel at the B8 T4096 H64 d64
    shape (bf16, no initial state, final state written)."""
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    B, T, H, D = 8, 4096, 64, 64
    print(f"[bench] generating Gated DeltaNet workload B{B} T{T} H{H} d{D}", file=sys.stderr, flush=True)
    inp = synth.make_gdn(B, T, H, D, seed=1301)
    names = ("q", "k", "v", "g", "beta")
    dev = {n: synth.to_torch(inp[n], "bf16", "cuda") for n in names}
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    sf = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ms = _time_launches(lambda i: wkv7.gdn_fwd(*(dev[n] for n in names), out=o, final_state=sf),
                        steps, warmup)
    cpu_rate = None
    if cpu:
        import numpy as np
        import oracle

        def call(sel):
            gsel = lambda x: np.stack([x[bb, :, h] for bb, h in sel])[:, :, None]
            oracle.gdn_fwd(*(gsel(inp[n]) for n in names), None)
        print("[bench] timing the CPU oracle (Gated DeltaNet) on a sample", file=sys.stderr, flush=True)
        cpu_rate = oracle_sample_rate(call, B, H, T)
    # q, k, v and o once (D channels each), g and beta once (one element per
    # token and head), the final state written once
    nbytes = 4 * B * T * H * D * 2 + 2 * B * T * H * 2 + B * H * D * D * 4
    name = f"gdn_fwd_bf16_B{B}_T{T}_H{H}_d{D}"
    return {name: {"ms": round(ms, 5), "Mtokens_per_s": round(B * T / ms / 1e3, 3),
                   "GB_per_s": round(nbytes / ms / 1e6, 1),
                   "frac_of_8TBps": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
                   "kernel": "chunked d64 (Gated DeltaNet)", "cpu_oracle": cpu_rate}}


def bwd_workload(steps, warmup, idx, cpu=True):
    """Backward (wkv7_bwd) on a forward workload's shape and inputs, with a
    seeded N(0, 1) output gradient rounded to bf16; the initial state and the
    mask of the workload are used, no final-state gradient."""
    import numpy as np
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    wl = synth.WORKLOADS[idx]
    B, T, H, D = wl["B"], wl["T"], wl["H"], wl["K"]
    print(f"[bench] generating backward workload on {wl['name']}", file=sys.stderr, flush=True)
    inp = synth.make(idx)
    names = ("r", "w", "k", "v", "a", "b")
    dev = {n: synth.to_torch(inp[n], "bf16", "cuda") for n in names}
    s0 = None if inp["s0"] is None else torch.from_numpy(inp["s0"]).cuda()
    mask = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).cuda()
    rng = np.random.default_rng(1400 + idx)
    d_o_np = synth.round_to(rng.standard_normal((B, T, H, D), dtype=np.float32), "bf16")
    d_o = synth.to_torch(d_o_np, "bf16", "cuda")
    cpu_rate = None
    if cpu:
        import oracle

        def call(sel):
            gsel = lambda x: np.stack([x[bb, :, h] for bb, h in sel])[:, :, None, :]
            s0s = None if inp["s0"] is None else np.stack([inp["s0"][bb, h] for bb, h in sel])[:, None]
            ms = None if inp["mask"] is None else np.stack([inp["mask"][bb] for bb, h in sel])
            oracle.bwd(*(gsel(inp[n]) for n in names), gsel(d_o_np), s0s, ms, None)
        print("[bench] timing the CPU oracle backward on a sample", file=sys.stderr, flush=True)
        cpu_rate = oracle_sample_rate(call, B, H, T)
    del inp, d_o_np
    ws = torch.empty(wkv7.bwd_workspace_bytes(B, T, H, D, D), dtype=torch.uint8, device="cuda")
    ms = _time_launches(lambda i: wkv7.bwd(*(dev[n] for n in names), d_o, initial_state=s0, mask=mask,
                                           workspace=ws), max(3, steps // 4), max(1, warmup // 4))
    tok = B * T * H * D * 2
    st = B * H * D * D * 4
    # inputs and d_o read once, six gradients written once, the initial
    # state read (if any) and its gradient written, the mask once
    nbytes = 7 * tok + 6 * tok + (st if s0 is not None else 0) + st + (B * T if mask is not None else 0)
    name = "bwd_" + wl["name"].replace("fwd_", "")
    return {name: {"ms": round(ms, 4), "Mtokens_per_s": round(B * T / ms / 1e3, 3),
                   "GB_per_s": round(nbytes / ms / 1e6, 1),
                   "frac_of_8TBps": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
                   "roofline": bwd_mfma_roofline(B, T, H, D, ms),
                   "workspace_bytes": ws.numel(),
                   "kernel": f"recurrences + per-chunk gradients, d{D}", "cpu_oracle": cpu_rate}}


FP32_MFMA_PEAK_TFLOPS = 157.3


def bwd_flops(B, T, H, D, L=16):
    """Matrix flops of the backward in chunk form: per 16-token chunk the
    forward chain (3 L D^2 + 4 L^2 D multiply-adds), the reverse chain
    (3 L D^2 + 4 L^2 D) and the per-chunk gradients (7 L D^2 + 22 L^2 D)."""
    nck = B * H * ((T + L - 1) // L)
    return 2 * nck * (13 * L * D * D + 30 * L * L * D)


def bwd_mfma_roofline(B, T, H, D, ms):
    """The backward computes in fp32 on the fp32 matrix cores: its bound is
    their dense peak, not HBM."""
    fl = bwd_flops(B, T, H, D)
    tf = fl / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "unit": "TFLOP/s", "peak": FP32_MFMA_PEAK_TFLOPS, "achieved": round(tf, 2),
            "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4), "flops": fl, "dtype": "f32",
            "note": "chunk-form matrix flops (13 L D^2 + 30 L^2 D multiply-adds per 16-token chunk)"}


def gdn_bwd_workload(steps, warmup, cpu=True):
    """Gated DeltaNet backward (wkv7_gdn_bwd) at the B8 T4096 H64 d64 shape
    (bf16, no initial state), seeded N(0, 1) output gradient rounded to
    bf16, no final-state gradient."""
    import numpy as np
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    B, T, H, D = 8, 4096, 64, 64
    print(f"[bench] generating Gated DeltaNet backward workload B{B} T{T} H{H} d{D}", file=sys.stderr, flush=True)
    inp = synth.make_gdn(B, T, H, D, seed=1301)
    names = ("q", "k", "v", "g", "beta")
    dev = {n: synth.to_torch(inp[n], "bf16", "cuda") for n in names}
    rng = np.random.default_rng(1501)
    d_o_np = synth.round_to(rng.standard_normal((B, T, H, D), dtype=np.float32), "bf16")
    d_o = synth.to_torch(d_o_np, "bf16", "cuda")
    cpu_rate = None
    if cpu:
        import oracle

        def call(sel):
            g3 = lambda x: np.stack([x[bb, :, h] for bb, h in sel])[:, :, None]
            oracle.gdn_bwd(*(g3(inp[n]) for n in names), g3(d_o_np))
        print("[bench] timing the CPU oracle (Gated DeltaNet backward) on a sample", file=sys.stderr, flush=True)
        cpu_rate = oracle_sample_rate(call, B, H, T)
    del inp, d_o_np
    ws = torch.empty(wkv7.gdn_bwd_workspace_bytes(B, T, H, D, D), dtype=torch.uint8, device="cuda")
    ms = _time_launches(lambda i: wkv7.gdn_bwd(*(dev[n] for n in names), d_o, workspace=ws),
                        max(3, steps // 4), max(1, warmup // 4))
    tok, tok1 = B * T * H * D * 2, B * T * H * 2
    # q, k, v, d_o and g, beta read once; dq, dk, dv and dg, dbeta written once;
    # the initial-state gradient written
    nbytes = 4 * tok + 2 * tok1 + 3 * tok + 2 * tok1 + B * H * D * D * 4
    name = f"gdn_bwd_bf16_B{B}_T{T}_H{H}_d{D}"
    return {name: {"ms": round(ms, 4), "Mtokens_per_s": round(B * T / ms / 1e3, 3),
                   "GB_per_s": round(nbytes / ms / 1e6, 1),
                   "frac_of_8TBps": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
                   "roofline": bwd_mfma_roofline(B, T, H, D, ms),
                   "workspace_bytes": ws.numel(),
                   "kernel": "recurrences + per-chunk gradients in Gated DeltaNet mode, d64",
                   "cpu_oracle": cpu_rate}}


def _time_launches(fn, steps, warmup):
    import torch
    settle(lambda: fn(0))
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def small_latency(steps, warmup, cpu=True):
    """Launch latency of the two small forward shapes (B1 T64 H1 d64 fp32;
    B2 T1024 H4 d64 bf16 with initial state and mask), which hold too few
    sequences to fill the GPU: reported as time per call under AUTO."""
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    out = {}
    for idx in (0, 1):
        wl = synth.WORKLOADS[idx]
        B, T, H, D, dt = wl["B"], wl["T"], wl["H"], wl["K"], wl["dtype"]
        inp = synth.make(idx)
        dev = {n: synth.to_torch(inp[n], dt, "cuda") for n in ("r", "w", "k", "v", "a", "b")}
        s0 = None if inp["s0"] is None else torch.from_numpy(inp["s0"]).cuda()
        mask = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).cuda()
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        o = torch.empty((B, T, H, D), dtype=tdt, device="cuda")
        sf = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
        ms = _time_launches(lambda i: wkv7.fwd(*(dev[n] for n in ("r", "w", "k", "v", "a", "b")),
                                               initial_state=s0, mask=mask, out=o, final_state=sf),
                            max(20, steps), warmup)
        path = wkv7.fwd_path(tdt, B, T, H, D, D)
        out[wl["name"]] = {"us_per_call": round(ms * 1e3, 2), "Mtokens_per_s": round(B * T / ms / 1e3, 3),
                           "kernel": "chunked" if path == wkv7.ALGO_CHUNKED else "recurrent",
                           "note": "latency only: too few sequences to fill the GPU"}
        if cpu:
            import oracle
            oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
            t0 = time.perf_counter()
            n = 0
            while time.perf_counter() - t0 < 0.5:
                oracle.fwd(*(inp[x] for x in ("r", "w", "k", "v", "a", "b")), inp["s0"], inp["mask"])
                n += 1
            dt = (time.perf_counter() - t0) / n
            out[wl["name"]]["cpu_oracle"] = {"us_per_call": round(dt * 1e6, 1), "kind": "oracle",
                                             "cores": min(16, len(os.sched_getaffinity(0))),
                                             "sample": f"the whole workload, {n} calls"}
        del dev, s0, mask, o, sf, inp
    return out


def fp32_workload(steps, warmup):
    """fp32 I/O at the workload-2 shape, B8 T4096 H64 d64, on both kernels.
    The chunked kernel (AUTO) runs the chunk form on the fp32 matrix cores:
    2 (8 L D + 4 D^2) flops per token and head at L = 16, 27 flop per HBM
    byte, above the fp32-matrix ridge (157.3 TFLOP/s / 8 TB/s = 20 flop/B),
    so it is reported against the fp32 matrix peak.  The recurrent kernel
    does 9 D^2 vector flops per token and head and is reported against the
    fp32 vector peak."""
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    wl = synth.WORKLOADS[2]
    B, T, H, D = wl["B"], wl["T"], wl["H"], wl["K"]
    print("[bench] generating the fp32 workload", file=sys.stderr, flush=True)
    inp = synth.make(2)
    dev = {n: synth.to_torch(inp[n], "f32", "cuda") for n in ("r", "w", "k", "v", "a", "b")}
    o = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
    sf = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    nbytes = algorithmic_bytes(B, T, H, D, 4, False, True, False)
    out = {}
    for algo, kind in ((wkv7.ALGO_AUTO, "chunked"), (wkv7.ALGO_RECURRENT, "recurrent")):
        ms = _time_launches(lambda i: wkv7.fwd(*(dev[n] for n in ("r", "w", "k", "v", "a", "b")), out=o,
                                               final_state=sf, algo=algo), max(3, steps // 5), warmup)
        if kind == "chunked":
            assert wkv7.fwd_path(torch.float32, B, T, H, D, D) == wkv7.ALGO_CHUNKED
            flops = 2 * (8 * 16 * D + 4 * D * D) * B * T * H
            roof = {"bound": "mfma", "unit": "TFLOP/s", "peak": FP32_MFMA_PEAK_TFLOPS, "dtype": "f32",
                    "note": "chunk-form flops, 2 (8 L D + 4 D^2) per token and head"}
            peak = FP32_MFMA_PEAK_TFLOPS
        else:
            flops = 9 * B * T * H * D * D
            roof = {"bound": "alu", "unit": "TFLOP/s", "peak": FP32_VECTOR_PEAK_TFLOPS,
                    "note": "9 K V vector flops per token and head"}
            peak = FP32_VECTOR_PEAK_TFLOPS
        roof.update({"achieved": round(flops / ms / 1e9, 2), "frac": round(flops / ms / 1e9 / peak, 4),
                     "flops": flops})
        out[f"fwd_f32_B{B}_T{T}_H{H}_d{D}_{kind}"] = {
            "ms": round(ms, 4), "Mtokens_per_s": round(B * T / ms / 1e3, 3), "GB_per_s": round(nbytes / ms / 1e6, 1),
            "frac_of_8TBps": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
            "roofline": roof, "kernel": f"{kind} d64 (fp32 I/O)"}
    del dev, o, sf, inp
    return out


def other_workloads(steps, warmup, cpu=True):
    """Latency of the two small forward shapes, the fp32 forward (chunked
    and recurrent) at the B8 T4096 H64 d64 shape, the packed variable-length forward, Gated
    DeltaNet (B8 T4096 H64 d64), the backward on the d64 and d128 shapes,
    the Gated DeltaNet backward and the Gated DeltaNet decode step (B512 H40
    d64, 256 consecutive in-place steps).  The d128 forward and the WKV7
    decode are in every bench line (d128_entry, decode_entry)."""
    import torch
    from rwkv_linear_attention_amd import synth, wkv7
    out = small_latency(steps, warmup, cpu)
    out.update(fp32_workload(steps, warmup))
    torch.cuda.empty_cache()
    out.update(varlen_workload(steps, warmup))
    torch.cuda.empty_cache()
    out.update(gdn_workload(steps, warmup, cpu))
    torch.cuda.empty_cache()
    out.update(bwd_workload(steps, warmup, 2, cpu))
    torch.cuda.empty_cache()
    out.update(bwd_workload(steps, warmup, 3, cpu))
    torch.cuda.empty_cache()
    out.update(gdn_bwd_workload(steps, warmup, cpu))
    torch.cuda.empty_cache()

    wl = synth.WORKLOADS[4]
    B, NSTEP, H, D = wl["B"], wl["T"], wl["H"], wl["K"]
    # Gated DeltaNet decode on the same shape: 256 consecutive in-place steps
    names = ("q", "k", "v", "g", "beta")
    print(f"[bench] generating Gated DeltaNet decode B{B} H{H} d{D} (32 distinct steps, cycled)",
          file=sys.stderr, flush=True)
    gin = synth.make_gdn(B, 32, H, D, seed=1302, init=True)
    gdev = {n: synth.to_torch(gin[n], "bf16", "cuda") for n in names}
    gsteps = [{n: gdev[n][:, t].contiguous() for n in names} for t in range(32)]
    gstate0 = torch.from_numpy(gin["s0"]).cuda()
    gstate = gstate0.clone()
    gbuf = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")

    def grun(i):
        gstate.copy_(gstate0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(NSTEP):
            x = gsteps[t % 32]
            wkv7.gdn_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state=gstate, out=gbuf)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    settle(lambda: wkv7.gdn_step(gsteps[0]["q"], gsteps[0]["k"], gsteps[0]["v"], gsteps[0]["g"],
                                 gsteps[0]["beta"], state=gstate, out=gbuf))
    grun(0)
    ms_total = min(grun(i) for i in range(3))
    gbytes = 2 * B * H * D * D * 4 + 3 * B * H * D * 2 + 2 * B * H * 2 + B * H * D * 2
    out[f"gdn_step_bf16_B{B}_H{H}_d{D}_x{NSTEP}"] = {
        "ms_256_steps": round(ms_total, 4), "us_per_step": round(ms_total * 1e3 / NSTEP, 2),
        "GB_per_s": round(gbytes * NSTEP / ms_total / 1e6, 1),
        "frac_of_8TBps": round(gbytes * NSTEP / ms_total / 1e6 / HBM_PEAK_GBS, 4),
        "bytes_per_step": gbytes, "kernel": "step d64 (Gated DeltaNet)",
        "note": "inputs of 32 distinct steps cycled; state reset outside the timed region"}
    return out


if __name__ == "__main__":
    main()

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
PROFILE_NOTE = os.path.join(ROOT, "profiles", "wkv7_chunked_B8_T4096_H64_d64.md")
KERNEL_SOURCES = [os.path.join(ROOT, "rwkv_linear_attention_amd", "csrc", f)
                  for f in ("wkv7_chunked.hip", "wkv7_common.hpp")]


def kernel_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(B, T, H, D, dtype_bytes, has_s0, has_final, has_mask):
    """Inputs once (r, w, k, v, a, b), o once, states once, mask 1 B/token."""
    tok = B * T * H * D * dtype_bytes
    st = B * H * D * D * 4
    return 6 * tok + tok + (st if has_s0 else 0) + (st if has_final else 0) + (B * T if has_mask else 0)


def measured_traffic(sha, launches_per_step=1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on this exact kernel source; otherwise None."""
    if not os.path.exists(PROFILE_NOTE):
        return None
    txt = open(PROFILE_NOTE).read()
    m = re.search(r"traffic: source_sha=(\w+) fetch_kib=([\d.]+) write_kib=([\d.]+) scale=([\d.]+)", txt)
    if not m or m.group(1) != sha:
        return None
    fetch, write, scale = float(m.group(2)), float(m.group(3)), float(m.group(4))
    return (fetch + write) * 1024.0 * scale / launches_per_step


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
    return {"value": full_tokens / t_used / 1e6, "unit": "Mtokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} (b,h) sequences of T={T} ({done / len(pairs):.2f} passes over the "
                      f"{len(pairs)} sequences of the workload; fp64 C, OpenMP), {t_used:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the operator is independent per (batch, head), "
              "so N GPUs run N disjoint batch/head shards with no communication; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rwkv_linear_attention_amd import synth, wkv7

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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record()
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
    t_all1.record()
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    launch_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / args.steps
    ms_per_step = total_ms / args.steps

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
    if not args.no_cpu:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, H, T)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Throughput of the heterogeneous-adapter LoRA apply on one MI355X.

Default workload: Llama-7B decode BGMV -- 64 tokens (one per request), the
q/k/v/o projections (4096 -> 4096) of one layer, 1000 rank-16 fp16 adapters
scattered over a unified page pool.  A step applies every token's adapter to
all four projections: y_i += s_a B_a (A_a x_i), shrink and expand fused in one
launch (lora_bgmv_apply).  16 different id batches (with their own x and y
buffers) rotate, so adapter pages come from HBM rather than the 256 MB
Infinity Cache.

`--workload` runs one of the other synthetic workloads the same way (for
profiling; the default is the measured configuration): the heterogeneous
decode batch (lora_bgmv_apply over its two slices) or a planned batch
(lora_apply over all slices; plans are built before the timed region).

Prints one JSON line.  `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BGMV/SGMV tokens/s and achieved HBM GB/s (% of peak), Llama-7B/70B shapes, 1 GPU"
HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(wl, ids: np.ndarray, slices, elt_y: int) -> int:
    """Bytes the method must move for one step: each distinct adapter's A and B
    once per slice, x once, y read and written once."""
    elt = 4 if wl.dtype == "f32" else 2
    total = 0
    uniq = sorted(set(int(a) for a in ids.tolist() if a >= 0))
    n = len(ids)
    for s in slices:
        d_in, d_out = wl.slices[s]
        for a in uniq:
            total += int(wl.ranks[a]) * (d_in + d_out) * elt
        total += n * d_in * elt + 2 * n * d_out * elt_y
    return total


# The sources the decode kernel (k_bgmv_apply) is compiled from.
DECODE_SOURCES = ("k_bgmv.hip", "kcommon.h", "kvalu.h", "lora_internal.h")


def kernel_source_hash() -> str:
    """Hash of the decode kernel's sources, so counter figures taken on other
    code are dropped."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gather_lora_matmul_amd", "csrc")
    paths = [os.path.join(csrc, f) for f in DECODE_SOURCES]
    paths.append(os.path.join(ROOT, "include", "lora_mi355x.h"))
    for path in paths:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the fused decode kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None if the kernel sources
    changed since the counters were taken."""
    prof = os.path.join(ROOT, "profiles", "bgmv_apply_llama7b_decode_traffic.json")
    try:
        with open(prof) as f:
            tj = json.load(f)
    except (OSError, ValueError):
        return None
    if tj.get("kernel_source_hash") != kernel_source_hash():
        return None
    return tj.get("hbm_bytes_per_launch")


def cpu_baseline(wl, batches, slices, threads: int, min_s: float = 10.0):
    """The fp64 oracle on the host, over whole batches of the same workload,
    repeated until at least `min_s` seconds of CPU work have been timed."""
    import oracle
    t0 = time.perf_counter()
    ntok = 0
    calls = 0
    while True:
        for b in batches:
            for s in slices:
                oracle.workload_reference(wl, b, s, n_threads=threads)
            ntok += len(b.ids)
            calls += 1
            if time.perf_counter() - t0 >= min_s:
                break
        if time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d batches of this workload (%d distinct) x %d slices = %d tokens, "
                      "fp64 C oracle, %.1f s" % (calls, len(batches), len(slices), ntok, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["fused", "split"], default="fused")
    ap.add_argument("--workload", default="llama7b_decode_bgmv",
                    choices=["llama7b_decode_bgmv", "hetero_decode_bgmv", "llama13b_prefill_sgmv",
                             "llama70b_mixed_apply"])
    ap.add_argument("--batches", type=int, default=None,
                    help="rotating batches (default 16 for decode, 4 for planned batches)")
    ap.add_argument("--planned", action="store_true",
                    help="decode workloads: plan each batch on the host and run lora_apply "
                         "(the SGMV path) instead of lora_bgmv_apply")
    ap.add_argument("--l-long", type=int, default=0,
                    help="planned batches: groups shorter than this run as short VALU items "
                         "(0: every group of a 16-bit pool is an MFMA tile)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 64 MiB device copy 10x (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this LoRA-apply path runs on a single GPU; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import gather_lora_matmul_amd as L
    import workloads as W
    from gather_lora_matmul_amd.synthetic import SyntheticPool, to_device

    torch.cuda.set_device(0)
    cfg = {"llama7b_decode_bgmv": 1, "hetero_decode_bgmv": 2, "llama13b_prefill_sgmv": 3,
           "llama70b_mixed_apply": 4}[args.workload]
    wl = W.make_workload(cfg)
    planned = cfg >= 3 or args.planned
    slices = list(range(len(wl.slices)))
    n_batches = args.batches or (4 if planned else 16)
    print("[bench] building pool: %s, %d adapters x %d slices" % (wl.name, wl.n_adapters, len(slices)),
          file=sys.stderr, flush=True)
    sp = SyntheticPool(wl)
    batches = [W.make_batch(wl, i) for i in range(n_batches)]
    ids_d = [torch.from_numpy(b.ids).cuda() for b in batches]
    xs = [[to_device(b.x[s], wl.dtype) for s in slices] for b in batches]
    ys = [[to_device(b.y0[s], wl.dtype) for s in slices] for b in batches]
    ydt = W.DTYPE_CODE[wl.dtype]
    n = len(batches[0].ids)
    v = [torch.zeros((n, sp.max_rank), dtype=torch.float32, device="cuda") for _ in slices]
    plans = []
    plan_host = {}
    if planned:
        t_build = []
        for b in batches:
            p = L.lora_plan_create(sp.handle, len(b.ids))
            t = time.perf_counter()
            L.lora_plan_build(p, b.ids, args.l_long)
            t_build.append(time.perf_counter() - t)
            plans.append(p)
        plan_host["plan_build_us"] = float(np.median(t_build)) * 1e6
    stream = torch.cuda.current_stream()

    def step(i):
        k = i % len(batches)
        io = [(s, xs[k][j], ys[k][j]) for j, s in enumerate(slices)]
        if planned:
            if args.mode == "fused":
                L.lora_apply(sp.handle, plans[k], io, ydt, stream=stream)
            else:
                for j, s in enumerate(slices):
                    L.lora_sgmv_shrink(sp.handle, plans[k], s, xs[k][j], v[j], stream=stream)
                    L.lora_sgmv_expand(sp.handle, plans[k], s, v[j], ys[k][j], ydt, stream=stream)
        elif args.mode == "fused":
            L.lora_bgmv_apply(sp.handle, io, ids_d[k], ydt, stream=stream)
        else:
            for j, s in enumerate(slices):
                L.lora_bgmv_shrink(sp.handle, s, xs[k][j], ids_d[k], v[j], stream=stream)
                L.lora_bgmv_expand(sp.handle, s, v[j], ids_d[k], ys[k][j], ydt, stream=stream)

    if planned:
        # host time of a plan's first launch (it builds the block ranges of the
        # launch shape) and of a later launch (ranges cached); untimed
        t_first, t_cached = [], []
        for k in range(len(batches)):
            torch.cuda.synchronize()
            t = time.perf_counter()
            step(k)
            t_first.append(time.perf_counter() - t)
            t = time.perf_counter()
            step(k)
            t_cached.append(time.perf_counter() - t)
        torch.cuda.synchronize()
        plan_host["first_launch_host_us"] = float(np.median(t_first)) * 1e6
        plan_host["cached_launch_host_us"] = float(np.median(t_cached)) * 1e6
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: wall clock over exactly K steps, bracketed by HIP events on
    # the stream the kernels are launched on (average launch duration =
    # event time / K; one launch per step in the fused mode)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = np.array([e0.elapsed_time(e1) / args.steps])
    ms_per_step = wall * 1e3 / args.steps
    toks = n * args.steps / wall
    elt_y = 2
    step_bytes = [algorithmic_bytes(wl, b.ids, slices, elt_y) for b in batches]
    used = [step_bytes[(args.warmup + i) % len(batches)] for i in range(args.steps)]
    avg_bytes = float(np.mean(used))
    avg_kernel_s = float(np.mean(kern_ms)) * 1e-3
    achieved = avg_bytes / avg_kernel_s / 1e9
    traffic = measured_traffic() if args.mode == "fused" and cfg == 1 and not planned else None
    if args.copy_calib:
        src = torch.empty(64 << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
    out = {
        "metric": METRIC,
        "value": toks,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens_per_step": n,
                   "slices": ", ".join("%dx%d" % tuple(d) for d in wl.slices),
                   "adapters": wl.n_adapters,
                   "rank": sorted(set(int(r) for r in wl.ranks)) if cfg != 1 else 16,
                   "weights": "%s N(0,0.02), pages scattered" % wl.dtype,
                   "entry": ("lora_apply" if planned else "lora_bgmv_apply") if args.mode == "fused"
                   else ("lora_sgmv_shrink+expand" if planned else "lora_bgmv_shrink+expand"),
                   "id_batches_rotated": len(batches)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "kernel_us_per_step": float(np.mean(kern_ms)) * 1e3,
        "algorithmic_MB_per_step": avg_bytes / 1e6,
        "kernel_source_hash": kernel_source_hash(),
        "accumulate": "f32",
    }
    if plan_host:
        out["plan_host_us"] = plan_host  # median per batch; host wall clock, outside the timed region
    if not args.no_cpu:
        threads = min(16, os.cpu_count() or 1)
        out["cpu_baseline"] = cpu_baseline(wl, batches, slices, threads)
    for p in plans:
        L.lora_plan_destroy(p)
    sp.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

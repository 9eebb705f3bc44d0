"""Throughput of the heterogeneous-adapter LoRA apply on one MI355X.

Headline workload: Llama-7B decode BGMV -- 64 tokens (one per request), the
q/k/v/o projections (4096 -> 4096) of one layer, 1000 rank-16 fp16 adapters
scattered over a unified page pool.  A step applies every token's adapter to
all four projections: y_i += s_a B_a (A_a x_i), shrink and expand fused in one
launch (lora_bgmv_apply).  16 different id batches (with their own x and y
buffers) rotate, so adapter pages come from HBM rather than the 256 MB
Infinity Cache.

The same run then times the other workloads of the metric (unless
--no-extra), each under `workloads` in the JSON line with its own algorithmic
bytes and roofline fraction: the heterogeneous decode batch through
lora_bgmv_apply and through a host plan (lora_apply), the Llama-13B prefill
SGMV batch and the Llama-70B-shape mixed batch (lora_apply on MFMA tiles), plus
a plain device copy and a streaming read as the measured bandwidth ceiling.

`--workload` makes another workload the headline (for profiling runs).
Prints one JSON line.  `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BGMV/SGMV tokens/s and achieved HBM GB/s (% of peak), Llama-7B/70B shapes, 1 GPU"
HBM_PEAK_GBS = 8000.0
WORKLOADS = {"llama7b_decode_bgmv": 1, "hetero_decode_bgmv": 2, "llama13b_prefill_sgmv": 3,
             "llama70b_mixed_apply": 4, "llama7b_decode_bgmv_fp8": 5}
ELT = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
CSRC = os.path.join(ROOT, "gather_lora_matmul_amd", "csrc")
# Sources each path's kernels are compiled from (traffic figures taken on other
# code are dropped).
BGMV_SOURCES = ("k_bgmv.hip", "kcommon.h", "kvalu.h", "lora_internal.h")
PLANNED_SOURCES = ("k_sgmv.hip", "kmfma.h", "kcommon.h", "kvalu.h", "lora_internal.h",
                   "layout.cpp", "plan.cpp")
DEVPLAN_SOURCES = ("k_devplan.hip", "devplan.h", "k_sgmv.hip", "kmfma.h", "kcommon.h", "kvalu.h",
                   "lora_internal.h")


def entry_of(planned: bool, devplan: bool, mode: str, reuse: bool = False) -> str:
    if devplan:
        return "lora_dplan_apply" if reuse else "lora_bgmv_apply_planned"
    if mode == "fused":
        return "lora_apply" if planned else "lora_bgmv_apply"
    return "lora_sgmv_shrink+expand" if planned else "lora_bgmv_shrink+expand"


def sources_of(planned: bool, devplan: bool):
    return DEVPLAN_SOURCES if devplan else (PLANNED_SOURCES if planned else BGMV_SOURCES)


def algorithmic_bytes(wl, ids: np.ndarray, slices, elt_y: int, shared_x: bool = False) -> int:
    """Bytes the method must move for one step: each distinct adapter's A and B
    once per slice (FP8 pages: one byte per code plus the 2 r fp32 scales), x
    once (once for all slices when they read one x), y read and written once."""
    elt, elt_x = ELT[wl.dtype], ELT[wl.act_dtype]
    total = 0
    uniq = sorted(set(int(a) for a in ids.tolist() if a >= 0))
    n = len(ids)
    for j, s in enumerate(slices):
        d_in, d_out = wl.slices[s]
        for a in uniq:
            r = int(wl.ranks[a])
            total += r * (d_in + d_out) * elt + (8 * r if wl.quantized else 0)
        total += (0 if shared_x and j > 0 else n * d_in * elt_x) + 2 * n * d_out * elt_y
    return total


def source_hash(files) -> str:
    h = hashlib.sha256()
    paths = [os.path.join(CSRC, f) for f in files] + [os.path.join(ROOT, "include", "lora_mi355x.h")]
    for path in paths:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, entry: str, src_hash: str, path: str = None):
    """HBM bytes per step of `entry` on `workload` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (profiles/hbm_traffic.json), or None if
    there is none or the kernels' sources changed since it was taken."""
    try:
        with open(path or os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
            tj = json.load(f)
    except (OSError, ValueError):
        return None
    rec = tj.get("records", {}).get("%s/%s" % (workload, entry))
    if not rec or rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_step")


# rocprofv3 names of the kernels one step of each entry point runs
STEP_KERNELS = {"lora_bgmv_apply": ("lora::k_bgmv_apply",),
                "lora_apply": ("lora::k_apply_", "lora::k_sgmv_", "lora::k_short_"),
                "lora_bgmv_shrink+expand": ("lora::k_bgmv_shrink", "lora::k_bgmv_expand"),
                "lora_sgmv_shrink+expand": ("lora::k_sgmv_", "lora::k_apply_", "lora::k_short_"),
                "lora_bgmv_apply_planned": ("k_devplan", "lora::k_apply_"),
                "lora_dplan_apply": ("lora::k_apply_",)}
COPY_BYTES = 64 << 20  # the --copy-calib copy


def _counter_rows(run_dir: str, counter: str):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    if not rows:
        raise SystemExit("no %s records under %s" % (counter, run_dir))
    return rows


def record_traffic(fetch_dir: str, write_dir: str, workload: str, entry: str, src_hash: str,
                   commands, path: str = None) -> dict:
    """HBM bytes per step of `entry` from a FETCH_SIZE and a WRITE_SIZE
    rocprofv3 run of `bench.py --copy-calib` (KiB per dispatch), each counter
    scaled by what it reads for the 64 MiB copy of the same run; stored under
    "workload/entry" in profiles/hbm_traffic.json with the kernels' source hash."""
    per = {}
    factors = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(run_dir, counter)
        copies = sorted(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]
                        or "copy" in r["Kernel_Name"].lower() and "lora" not in r["Kernel_Name"])
        big = copies[-10:]
        if len(big) < 10 or big[0] < 0.25 * COPY_BYTES / 1024:
            raise SystemExit("%s: the 64 MiB copies of --copy-calib are missing" % run_dir)
        factors[counter] = COPY_BYTES / (float(np.median(big)) * 1024)
        for r in rows:
            name = r["Kernel_Name"]
            if any(k in name for k in STEP_KERNELS[entry]):
                per.setdefault(name, {}).setdefault(counter, []).append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit("no %s kernels in the counter records" % entry)
    kernels, total = {}, 0.0
    for name, c in sorted(per.items()):
        f = float(np.mean(c.get("FETCH_SIZE", [0.0])))
        w = float(np.mean(c.get("WRITE_SIZE", [0.0])))
        b = (f * factors["FETCH_SIZE"] + w * factors["WRITE_SIZE"]) * 1024
        kernels[name] = {"dispatches": len(c.get("FETCH_SIZE", [])), "fetch_KiB_mean": f,
                         "write_KiB_mean": w, "hbm_bytes": b}
        total += b
    path = path or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            tj = json.load(fh)
    except (OSError, ValueError):
        tj = {}
    tj["what"] = ("HBM bytes per step: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, two rocprofv3 "
                  "--pmc runs of bench.py --copy-calib) each scaled by the counter's reading for a "
                  "64 MiB device copy in the same run; mean over the step kernels' dispatches")
    rec = {"hbm_bytes_per_step": total, "kernel_source_hash": src_hash,
           "fetch_factor": factors["FETCH_SIZE"], "write_factor": factors["WRITE_SIZE"],
           "kernels": kernels, "commands": list(commands)}
    tj.setdefault("records", {})["%s/%s" % (workload, entry)] = rec
    with open(path, "w") as fh:
        json.dump(tj, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rate(wl, batches, slices, threads: int, min_s: float):
    """Tokens/s of the fp64 oracle over whole batches of the workload, repeated
    until at least `min_s` seconds of CPU work have been timed."""
    import oracle
    t0 = time.perf_counter()
    ntok = calls = 0
    while time.perf_counter() - t0 < min_s:
        b = batches[calls % len(batches)]
        for s in slices:
            oracle.workload_reference(wl, b, s, n_threads=threads)
        ntok += len(b.ids)
        calls += 1
    dt = time.perf_counter() - t0
    return ntok / dt, calls, ntok, dt


def cpu_baseline(wl, batches, slices):
    """The oracle as it stands on the host: all the threads this process may use
    (at most 16, the machine's CPU share for one GPU) and one thread."""
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    threads = max(1, min(16, allowed))
    rate, calls, ntok, dt = oracle_rate(wl, batches, slices, threads, 10.0)
    rate1, calls1, ntok1, dt1 = oracle_rate(wl, batches, slices, 1, 5.0)
    return {"value": rate, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d batches of this workload (%d distinct) x %d slices = %d tokens, fp64 C "
                      "oracle, %.1f s on %d threads" % (calls, len(batches), len(slices), ntok, dt,
                                                        threads),
            "value_1_thread": rate1,
            "sample_1_thread": "%d batches = %d tokens, %.1f s" % (calls1, ntok1, dt1),
            "host_cpus": os.cpu_count(), "affinity_cpus": allowed, "cpu_model": cpu_model()}


class Runner:
    """One workload set up for timing: pool, rotating batches, plans and
    workspaces, and the step that applies one batch."""

    def __init__(self, name: str, mode: str = "fused", planned: bool = False, n_batches=None,
                 l_long: int = 0, qkv=None, n_tokens=None, devplan: bool = False,
                 reuse: bool = False):
        """qkv: None, or "separate" / "shared": q, k and v (slices 0-2) reading
        one x buffer, without or with an x_group (decode BGMV only).  devplan:
        decode workloads through lora_bgmv_apply_planned (tokens grouped by
        adapter on the device); with reuse, each rotating batch's device plan is
        built once before timing and a step is lora_dplan_apply alone (the cost
        of every further layer that shares a decode step's ids)."""
        import torch

        import gather_lora_matmul_amd as L
        import workloads as W
        from gather_lora_matmul_amd.synthetic import SyntheticPool, prepare_shapes, to_device
        self.L, self.torch = L, torch
        cfg = WORKLOADS[name]
        self.wl = wl = W.make_workload(cfg)
        self.planned = planned or cfg in (3, 4)
        self.devplan = devplan and not self.planned
        self.reuse = self.devplan and reuse
        if self.devplan:
            mode = "fused"
        self.mode = mode
        self.qkv = qkv
        # traffic records exist only for the workloads' own batches
        self.traffic_ok = qkv is None and n_tokens is None
        self.slices = slices = [0, 1, 2] if qkv else list(range(len(wl.slices)))
        n_batches = n_batches or (4 if self.planned else 16)
        t0 = time.perf_counter()
        print("[bench] %s: pool of %d adapters x %d slices" % (name, wl.n_adapters, len(slices)),
              file=sys.stderr, flush=True)
        self.sp = SyntheticPool(wl)
        self.setup_s = time.perf_counter() - t0
        self.batches = [W.make_batch(wl, i, n_tokens=n_tokens) for i in range(n_batches)]
        self.ids_d = [torch.from_numpy(b.ids).cuda() for b in self.batches]
        if qkv:  # one x per batch for q, k and v
            for b in self.batches:
                b.x[1] = b.x[0]
                b.x[2] = b.x[0]
            self.xs = [[to_device(b.x[0], wl.act_dtype)] * 3 for b in self.batches]
        else:
            self.xs = [[to_device(b.x[s], wl.act_dtype) for s in slices] for b in self.batches]
        self.ys = [[to_device(b.y0[s], wl.act_dtype) for s in slices] for b in self.batches]
        self.ydt = W.DTYPE_CODE[wl.act_dtype]
        self.n = len(self.batches[0].ids)
        self.v = [torch.zeros((self.n, self.sp.max_rank), dtype=torch.float32, device="cuda")
                  for _ in slices]
        self.plans, self.wss, self.plan_host = [], [], {}
        if self.planned:
            t_build, t_prep = [], []
            shapes = [slices] if mode == "fused" else [[s] for s in slices]
            for b in self.batches:
                p = L.lora_plan_create(self.sp.handle, len(b.ids))
                t = time.perf_counter()
                L.lora_plan_build(p, b.ids, l_long)
                t_build.append(time.perf_counter() - t)
                t = time.perf_counter()
                self.wss.append(prepare_shapes(p, shapes))
                t_prep.append(time.perf_counter() - t)
                self.plans.append(p)
            torch.cuda.synchronize()
            self.plan_host["plan_build_us"] = float(np.median(t_build)) * 1e6
            self.plan_host["prepare_us"] = float(np.median(t_prep)) * 1e6
        self.stream = torch.cuda.current_stream()
        self.stream_h = self.stream.cuda_stream
        # fused steps: arguments checked and marshalled once per rotating batch
        self.calls = []
        self.ws_dev = None
        self.dplans = []
        if self.reuse:
            for k, b in enumerate(self.batches):
                d = L.lora_dplan_create(self.sp.handle, len(b.ids), slices)
                L.lora_dplan_build(d, slices, self.ids_d[k])
                self.dplans.append(d)
            torch.cuda.synchronize()
        elif self.devplan:
            n_max = max(len(b.ids) for b in self.batches)
            self.ws_dev = torch.empty(L.lora_bgmv_planned_workspace_size(self.sp.handle, slices, n_max),
                                      dtype=torch.uint8, device="cuda")
        if mode == "fused":
            for k, b in enumerate(self.batches):
                group = 1 if qkv == "shared" else 0
                io = [(s, self.xs[k][j], self.ys[k][j], group) for j, s in enumerate(slices)]
                if self.planned:
                    c = L.prepare_apply(self.sp.handle, self.plans[k], io, self.ydt, workspace=self.wss[k])
                elif self.reuse:
                    c = L.prepare_dplan_apply(self.sp.handle, self.dplans[k], io, len(b.ids), self.ydt)
                elif self.devplan:
                    c = L.prepare_bgmv_apply_planned(self.sp.handle, io, self.ids_d[k], self.ydt,
                                                     self.ws_dev)
                else:
                    c = L.prepare_bgmv_apply(self.sp.handle, io, self.ids_d[k], self.ydt)
                self.calls.append(c)
        self.entry = entry_of(self.planned, self.devplan, mode, self.reuse)
        self.src_hash = source_hash(sources_of(self.planned, self.devplan))

    def step(self, i: int):
        L, k = self.L, i % len(self.batches)
        if self.calls:  # fused: one prepared call
            self.calls[k](self.stream_h)
        elif self.planned:
            for j, s in enumerate(self.slices):
                L.lora_sgmv_shrink(self.sp.handle, self.plans[k], s, self.xs[k][j], self.v[j],
                                   workspace=self.wss[k], stream=self.stream)
                L.lora_sgmv_expand(self.sp.handle, self.plans[k], s, self.v[j],
                                   self.ys[k][j], self.ydt, stream=self.stream)
        else:
            for j, s in enumerate(self.slices):
                L.lora_bgmv_shrink(self.sp.handle, s, self.xs[k][j], self.ids_d[k], self.v[j],
                                   stream=self.stream)
                L.lora_bgmv_expand(self.sp.handle, s, self.v[j], self.ids_d[k], self.ys[k][j],
                                   self.ydt, stream=self.stream)

    def time(self, steps: int, warmup: int):
        """Wall clock over exactly `steps` steps, bracketed by HIP events on the
        stream the kernels are launched on."""
        torch = self.torch
        if self.planned:  # host time of one planned step (checks and launches), untimed
            t_launch = []
            for k in range(len(self.batches)):
                torch.cuda.synchronize()
                t = time.perf_counter()
                self.step(k)
                t_launch.append(time.perf_counter() - t)
            self.plan_host["launch_host_us"] = float(np.median(t_launch)) * 1e6
        for i in range(warmup):
            self.step(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(self.stream)
        for i in range(steps):
            self.step(warmup + i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        event_s = e0.elapsed_time(e1) * 1e-3 / steps
        used = [algorithmic_bytes(self.wl, self.batches[(warmup + i) % len(self.batches)].ids,
                                  self.slices, 2, shared_x=bool(self.qkv)) for i in range(steps)]
        return wall, event_s, float(np.mean(used))

    def record(self, steps: int, warmup: int):
        wall, event_s, avg_bytes = self.time(steps, warmup)
        achieved = avg_bytes / event_s / 1e9
        rec = {"entry": self.entry, "tokens_per_step": self.n, "steps": steps, "warmup": warmup,
               "tokens_per_s": self.n * steps / wall, "ms_per_step": wall * 1e3 / steps,
               "event_us_per_step": event_s * 1e6, "algorithmic_MB_per_step": avg_bytes / 1e6,
               "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                            "basis": "algorithmic bytes / (HIP-event time of the timed steps / "
                                     "steps), launch gaps included",
                            "traffic": (measured_traffic(self.wl.name, self.entry, self.src_hash)
                                        if self.traffic_ok else None)},
               "kernel_source_hash": self.src_hash, "pool_setup_s": self.setup_s}
        if self.plan_host:
            rec["plan_host_us"] = self.plan_host
        return rec

    def close(self):
        for p in self.plans:
            self.L.lora_plan_destroy(p)
        self.plans = []
        for d in self.dplans:
            self.L.lora_dplan_destroy(d)
        self.dplans = []
        self.sp.close()


def bandwidth_ceiling():
    """Measured device bandwidth of plain streaming kernels on 1 GiB buffers
    (beyond the 256 MB Infinity Cache): a device-to-device copy (read + write
    bytes) and a sum (read bytes)."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
        src.sum()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    for _ in range(10):
        dst.copy_(src)
    e[1].record()
    e[2].record()
    for _ in range(10):
        src.sum()
    e[3].record()
    torch.cuda.synchronize()
    copy_s = e[0].elapsed_time(e[1]) * 1e-3 / 10
    read_s = e[2].elapsed_time(e[3]) * 1e-3 / 10
    del src, dst
    return {"copy_GBs": 2 * 4 * n / copy_s / 1e9, "read_GBs": 4 * n / read_s / 1e9,
            "bytes": 4 * n, "kernels": "torch copy_ and sum over 1 GiB fp32, 10 calls each"}


def residency(n_set: int = 64, steps: int = 100):
    """On-demand residency on the Llama-7B decode shapes (4 slices, rank 16,
    fp16): a host store of 4 * n_set + 1 adapters, a pool with room for all of
    them; set A is resident and computed on, sets B1..B3 are loaded cold.
    Reports the upload rate of a cold set, the time until one rare adapter is
    usable, and how much of a load hides under compute already enqueued:
    overlap = (t_compute + t_upload - t_both) / min(t_compute, t_upload)."""
    import torch

    import gather_lora_matmul_amd as L
    import workloads as W
    from gather_lora_matmul_amd.synthetic import to_device
    wl = W.make_workload(1)
    n_ad = 4 * n_set + 1
    P = wl.page_elems
    per_adapter = sum(16 + -(-d_out // (P // 16)) for _, d_out in wl.slices)
    pool = L.lora_pool_create(P, L.LORA_F16, per_adapter * n_ad + 8, wl.n_adapters, 16, wl.slices,
                              shuffle_seed=wl.shuffle_seed, act_dtype=L.LORA_F16)
    L.lora_page_table_build(pool)
    store = L.lora_store_create(pool)
    t0 = time.perf_counter()
    for a in range(n_ad):
        for s in range(4):
            A, B = wl.weights(a, s)
            L.lora_store_add(store, a, s, 16, float(wl.scales[a]), A, B)
    reg_s = time.perf_counter() - t0
    up = torch.cuda.Stream()
    cs = torch.cuda.current_stream()
    sets = [np.arange(k * n_set, (k + 1) * n_set, dtype=np.int32) for k in range(4)]
    L.lora_store_ensure(store, sets[0], upload_stream=up, compute_stream=cs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    ids = torch.from_numpy(rng.choice(sets[0], size=64).astype(np.int32)).cuda()
    xs = [to_device(W.make_batch(wl, 0).x[s], "f16") for s in range(4)]
    ys = [torch.zeros((64, 4096), dtype=torch.float16, device="cuda") for _ in range(4)]
    call = L.prepare_bgmv_apply(pool, [(s, xs[s], ys[s]) for s in range(4)], ids, L.LORA_F16)
    sh = cs.cuda_stream
    for _ in range(10):
        call(sh)
    torch.cuda.synchronize()

    def compute():
        for _ in range(steps):
            call(sh)

    t = time.perf_counter()
    compute()
    torch.cuda.synchronize()
    t_c = time.perf_counter() - t
    bytes0 = L.lora_store_get_stats(store)["bytes_uploaded"]
    t = time.perf_counter()
    L.lora_store_ensure(store, sets[1], upload_stream=up, compute_stream=cs)
    torch.cuda.synchronize()
    t_u = time.perf_counter() - t
    set_bytes = L.lora_store_get_stats(store)["bytes_uploaded"] - bytes0
    t = time.perf_counter()
    compute()
    L.lora_store_ensure(store, sets[2], upload_stream=up, compute_stream=cs)
    torch.cuda.synchronize()
    t_both = time.perf_counter() - t
    t = time.perf_counter()
    L.lora_store_ensure(store, np.array([4 * n_set], np.int32), upload_stream=up, compute_stream=cs)
    torch.cuda.synchronize()
    t_one = time.perf_counter() - t
    st = L.lora_store_get_stats(store)
    L.lora_store_destroy(store)
    L.lora_pool_destroy(pool)
    return {"workload": "llama7b_decode_bgmv adapters (4 slices x rank 16, fp16: 1 MiB each)",
            "set_adapters": n_set, "set_MB": set_bytes / 1e6, "upload_GBs": set_bytes / t_u / 1e9,
            "upload_ms": t_u * 1e3, "compute_ms": t_c * 1e3, "both_ms": t_both * 1e3,
            "overlap": (t_c + t_u - t_both) / min(t_c, t_u),
            "one_adapter_ms": t_one * 1e3, "register_s": reg_s, "uploads": st["uploads"],
            "compute": "%d lora_bgmv_apply steps on resident adapters" % steps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["fused", "split"], default="fused")
    ap.add_argument("--workload", default="llama7b_decode_bgmv", choices=sorted(WORKLOADS))
    ap.add_argument("--batches", type=int, default=None,
                    help="rotating batches (default 16 for decode, 4 for planned batches)")
    ap.add_argument("--planned", action="store_true",
                    help="decode workloads: plan each batch on the host and run lora_apply "
                         "(the SGMV path) instead of lora_bgmv_apply")
    ap.add_argument("--devplan", action="store_true",
                    help="decode workloads: group the tokens by adapter on the device "
                         "(lora_bgmv_apply_planned) instead of lora_bgmv_apply")
    ap.add_argument("--reuse-plan", action="store_true",
                    help="with --devplan: build each batch's device plan once, time lora_dplan_apply")
    ap.add_argument("--l-long", type=int, default=0,
                    help="planned batches: groups shorter than this run as short VALU items "
                         "(0: every group of a 16-bit pool is an MFMA tile)")
    ap.add_argument("--tokens", type=int, default=None,
                    help="decode workloads: tokens per batch instead of the workload's own "
                         "(a profiling line, not the headline)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 64 MiB device copy 10x (HBM counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no timing: store the HBM bytes per step of --workload (and --planned) "
                         "from a FETCH_SIZE and a WRITE_SIZE rocprofv3 run into "
                         "profiles/hbm_traffic.json")
    ap.add_argument("--command", action="append", default=[],
                    help="with --record-traffic: the profiling commands, kept in the record")
    args = ap.parse_args()
    if args.record_traffic:
        cfg = WORKLOADS[args.workload]
        planned = args.planned or cfg in (3, 4)
        devplan = args.devplan and not planned
        entry = entry_of(planned, devplan, args.mode, args.reuse_plan)
        rec = record_traffic(args.record_traffic[0], args.record_traffic[1], args.workload, entry,
                             source_hash(sources_of(planned, devplan)), args.command)
        print(json.dumps({"workload": args.workload, "entry": entry,
                          "hbm_MB_per_step": rec["hbm_bytes_per_step"] / 1e6,
                          "fetch_factor": rec["fetch_factor"], "write_factor": rec["write_factor"]}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this LoRA-apply path runs on a single GPU; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    head = Runner(args.workload, args.mode, args.planned, args.batches, args.l_long,
                  n_tokens=args.tokens, devplan=args.devplan, reuse=args.reuse_plan)
    rec = head.record(args.steps, args.warmup)
    wl = head.wl
    cfg = WORKLOADS[args.workload]
    out = {
        "metric": METRIC,
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens_per_step": head.n,
                   "slices": ", ".join("%dx%d" % tuple(d) for d in wl.slices),
                   "adapters": wl.n_adapters,
                   "rank": sorted(set(int(r) for r in wl.ranks)) if cfg not in (1, 5) else 16,
                   "weights": "%s N(0,0.02), pages scattered" % wl.dtype,
                   "entry": head.entry, "id_batches_rotated": len(head.batches)},
        "roofline": rec["roofline"],
        "kernel_us_per_step": rec["event_us_per_step"],
        "algorithmic_MB_per_step": rec["algorithmic_MB_per_step"],
        "kernel_source_hash": rec["kernel_source_hash"],
        "accumulate": "f32",
    }
    if "plan_host_us" in rec:
        out["plan_host_us"] = rec["plan_host_us"]
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, head.batches, head.slices)
    if args.copy_calib:
        src = torch.empty(64 << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
    head.close()
    if not args.no_extra:
        extra = {}
        steps = min(args.steps, 50)
        warm = min(args.warmup, 5)
        for name, planned, qkv, ntok, dp in (("llama7b_decode_bgmv", False, "separate", None, False),
                                             ("llama7b_decode_bgmv", False, "shared", None, False),
                                             ("llama7b_decode_bgmv", False, "separate", 256, False),
                                             ("llama7b_decode_bgmv", False, "shared", 256, False),
                                             ("llama7b_decode_bgmv", False, None, None, True),
                                             ("llama7b_decode_bgmv_fp8", False, None, None, False),
                                             ("hetero_decode_bgmv", False, None, None, False),
                                             ("hetero_decode_bgmv", False, None, None, True),
                                             ("hetero_decode_bgmv", False, None, None, "reuse"),
                                             ("hetero_decode_bgmv", True, None, None, False),
                                             ("llama13b_prefill_sgmv", True, None, None, False),
                                             ("llama70b_mixed_apply", True, None, None, False)):
            key = name + ("/planned" if planned and WORKLOADS[name] in (1, 2) else "")
            key += "/device_plan_reused" if dp == "reuse" else ("/device_planned" if dp else "")
            key += "/qkv_%s_x" % qkv if qkv else ""
            key += "_%dtok" % ntok if ntok else ""
            if (name == args.workload and planned == head.planned and bool(dp) == head.devplan
                    and (dp == "reuse") == head.reuse and not qkv):
                continue
            r = Runner(name, "fused", planned, qkv=qkv, n_tokens=ntok, devplan=bool(dp),
                       reuse=dp == "reuse")
            extra[key] = r.record(steps, warm)
            r.close()
            print("[bench] %s: %.1f us per step, %.3f of 8 TB/s" % (
                key, extra[key]["event_us_per_step"], extra[key]["roofline"]["frac"]),
                file=sys.stderr, flush=True)
        out["workloads"] = extra
        out["residency"] = residency()
        print("[bench] residency: %.1f GB/s upload, overlap %.2f" % (
            out["residency"]["upload_GBs"], out["residency"]["overlap"]), file=sys.stderr, flush=True)
        out["bandwidth_ceiling"] = bandwidth_ceiling()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Per-block timeline of the fused decode launch (lora_bgmv_apply) on one of
the synthetic workloads, from the profiling build of the library.

    python gather_lora_matmul_amd/build.py --timeline
    python gather_lora_matmul_amd/timeline.py --workload hetero_decode_bgmv [--tokens N]

Each block of the launch records its start and end on the 100 MHz constant
clock, the compute unit its first wave ran on, and its (slice, token, rank,
row split); the summary gives block durations by (slice, rank), the number of
blocks running over time, and per compute unit the idle gaps between
consecutive blocks.  Compute units are told apart by the XCD (taken as block
index mod 8, the order in which the hardware hands out the blocks of a grid)
and the shader engine, shader array and compute unit fields of the wave id.
"""
from __future__ import annotations

import argparse
import collections
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TIMELINE_LIB = os.path.join(ROOT, "gather_lora_matmul_amd", "liblora_mi355x_timeline.so")


def summarize(rec: np.ndarray, title: str) -> str:
    r = rec[rec[:, 7] == 1].astype(np.int64)
    nb = len(r)
    base = r[:, 0].min()
    t0 = (r[:, 0] - base) / 100.0
    t1 = (r[:, 1] - base) / 100.0
    d = t1 - t0
    sl, rk = r[:, 3].astype(np.int32), r[:, 4]
    out = ["### %s" % title, "",
           "blocks %d, span %.1f us, last block start %.1f us, duration median %.1f us (max %.1f)"
           % (nb, t1.max(), t0.max(), np.median(d), d.max()), "",
           "| slice | rank | blocks | duration med / min / max (us) | start med / max (us) | end max (us) |",
           "|---|---|---|---|---|---|"]
    groups = collections.defaultdict(list)
    for i in range(nb):
        groups[(int(sl[i]), int(rk[i]))].append(i)
    for k in sorted(groups):
        ii = groups[k]
        out.append("| %d | %d | %d | %.1f / %.1f / %.1f | %.1f / %.1f | %.1f |" % (
            k[0], k[1], len(ii), np.median(d[ii]), d[ii].min(), d[ii].max(), np.median(t0[ii]),
            t0[ii].max(), t1[ii].max()))
    ts = np.linspace(0, t1.max(), 12)
    out += ["", "blocks running at %s us: %s" % (
        ", ".join("%.0f" % t for t in ts), ", ".join(str(int(((t0 <= t) & (t1 > t)).sum())) for t in ts))]
    hw = r[:, 2]
    idx = np.arange(nb)
    key = list(zip(idx % 8, (hw >> 13) & 3, (hw >> 12) & 1, (hw >> 8) & 15))
    cus = collections.defaultdict(list)
    for i, k in enumerate(key):
        cus[k].append(i)
    # per compute unit: the union of its blocks' intervals (blocks may overlap
    # when several are resident at once), the idle gaps between busy stretches
    gaps, idle_end, busy_t, conc = [], [], 0.0, 1
    for v in cus.values():
        v = sorted(v, key=lambda j: t0[j])
        cur_s, cur_e = t0[v[0]], t1[v[0]]
        for j in v[1:]:
            conc = max(conc, int(((t0[v] <= t0[j]) & (t1[v] > t0[j])).sum()))
            if t0[j] > cur_e:
                gaps.append(t0[j] - cur_e)
                busy_t += cur_e - cur_s
                cur_s, cur_e = t0[j], t1[j]
            else:
                cur_e = max(cur_e, t1[j])
        busy_t += cur_e - cur_s
        idle_end.append(t1.max() - cur_e)
    gaps = np.array(gaps) if gaps else np.zeros(1)
    per_cu = collections.Counter(len(v) for v in cus.values())
    busy = busy_t / (len(cus) * t1.max())
    out += ["compute units %d (blocks per unit: %s; at most %d at once); busy fraction %.2f" % (
                len(cus), ", ".join("%d: %d" % kv for kv in sorted(per_cu.items())), conc, busy),
            "idle gaps between busy stretches of one unit: median %.2f us, p90 %.2f, max %.2f; "
            "idle after its last block: median %.1f us" % (
                np.median(gaps), np.percentile(gaps, 90), gaps.max(), np.median(idle_end)), ""]
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="hetero_decode_bgmv")
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--runs", type=int, default=3)
    ap.add_argument("--lib", default=TIMELINE_LIB)
    args = ap.parse_args()
    os.environ["LORA_MI355X_LIB"] = args.lib
    sys.path.insert(0, ROOT)
    import torch
    import gather_lora_matmul_amd as L
    import workloads as W
    from gather_lora_matmul_amd.synthetic import SyntheticPool, to_device
    cfg = {v: k for k, v in W.CONFIG_NAMES.items()}[args.workload]
    wl = W.make_workload(cfg)
    b = W.make_batch(wl, 0, n_tokens=args.tokens)
    used = sorted(set(int(a) for a in b.ids if a >= 0))
    sp = SyntheticPool(wl, adapters=used)
    try:
        ids = torch.from_numpy(b.ids.astype(np.int32)).cuda()
        S = list(range(len(wl.slices)))
        xs = [to_device(b.x[s], wl.act_dtype) for s in S]
        ys = [to_device(b.y0[s], wl.act_dtype) for s in S]
        io = [(s, xs[s], ys[s]) for s in S]
        for _ in range(20):
            L.lora_bgmv_apply(sp.handle, io, ids, W.DTYPE_CODE[wl.act_dtype])
        torch.cuda.synchronize()
        print("# Fused decode per-block timeline: %s, %d tokens x %d slices, %d distinct adapters\n"
              % (args.workload, len(b.ids), len(S), len(used)))
        for k in range(args.runs):
            L.lora_debug_block_timeline(1)  # fails early on a build without the timeline
            L.lora_bgmv_apply(sp.handle, io, ids, W.DTYPE_CODE[wl.act_dtype])
            torch.cuda.synchronize()
            rec = L.lora_debug_block_timeline(65536)
            n_blocks = int(np.nonzero(rec[:, 7])[0].max()) + 1
            print(summarize(rec[:n_blocks], "launch %d" % (k + 1)), flush=True)
    finally:
        sp.close()


if __name__ == "__main__":
    main()

"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded workload batches and compare element by element with the fp64 oracle."""
from __future__ import annotations

import sys
from typing import Optional, Sequence

import numpy as np

import oracle
import workloads as W

REL_L2 = 1e-3          # relative L2 bound on the whole output of a call
MAX_ABS = 5e-3         # max |error| <= MAX_ABS * max |y_ref|
GUARD = 64             # canary elements before and after every output buffer


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def _gate(got: np.ndarray, cmp: np.ndarray, ref_scale: float, what: str):
    d = got - cmp
    nrm = np.linalg.norm(cmp)
    rel = np.linalg.norm(d) / nrm if nrm > 0 else np.linalg.norm(d)
    mx = np.abs(d).max() if d.size else 0.0
    bound = MAX_ABS * max(ref_scale, 1e-30)
    assert rel <= REL_L2, "%s: rel L2 %.3e > %.1e" % (what, rel, REL_L2)
    assert mx <= bound, "%s: max abs %.3e > %.3e" % (what, mx, bound)
    return rel, mx


def compare(y_gpu_bits: np.ndarray, y_ref: np.ndarray, y_dtype: str, what: str = "",
            y0_bits: Optional[np.ndarray] = None):
    """Gate A (fp32 y): against the unrounded fp64 result.  Gate B (16-bit y):
    against the oracle's result rounded once to the y dtype.  Every element of
    the call is compared.  With fp32 y and a non-zero y0 (given as y0_bits) the
    LoRA delta itself, y - y0, is also gated against the oracle's delta, so an
    error in the delta cannot hide under the norm of y0."""
    if y_dtype == "f32":
        cmp = y_ref
    else:
        cmp = oracle.decode(oracle.round_to(y_ref, y_dtype), y_dtype)
    g = W.dequantize(y_gpu_bits, y_dtype)
    assert g.shape == cmp.shape, (g.shape, cmp.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite output (poisoned page read?)" % what
    out = _gate(g, cmp, np.abs(y_ref).max() if y_ref.size else 0.0, what)
    if y0_bits is not None and y_dtype == "f32" and np.any(y0_bits != 0):
        y0 = W.dequantize(y0_bits, "f32")
        delta_ref = y_ref - y0
        _gate(g - y0, delta_ref, np.abs(delta_ref).max() if delta_ref.size else 0.0,
              what + " (delta y - y0)")
    return out


def compare_v(v_gpu: np.ndarray, v_ref: np.ndarray, ids: np.ndarray, ranks: np.ndarray,
              what: str = ""):
    """Split-API shrink output: v[i][k] for k < r_{a_i} within the gate of the
    oracle's v; exact zeros for r_{a_i} <= k < v_ld and for tokens without an
    adapter."""
    assert v_gpu.shape == v_ref.shape, (v_gpu.shape, v_ref.shape)
    n, v_ld = v_gpu.shape
    r = np.where(ids >= 0, ranks[np.clip(ids, 0, None)], 0)
    inside = np.arange(v_ld)[None, :] < r[:, None]
    assert np.all(v_gpu[~inside] == 0), "%s: v not zero past the rank (%d elements)" % (
        what, int(np.sum(v_gpu[~inside] != 0)))
    g = v_gpu.astype(np.float64)[inside]
    assert np.all(np.isfinite(g)), "%s: non-finite v" % what
    if g.size:
        _gate(g, v_ref[inside], np.abs(v_ref[inside]).max(), what + " (v)")


def exact_compare(y_gpu_bits: np.ndarray, y_ref: np.ndarray, y_dtype: str, what: str = ""):
    want = oracle.round_to(y_ref, y_dtype)
    if y_dtype == "f32":
        ok = np.array_equal(y_gpu_bits.view(np.uint32), want.view(np.uint32))
    else:
        ok = np.array_equal(y_gpu_bits, want)
    if not ok:
        bad = np.argwhere(y_gpu_bits != want)
        raise AssertionError("%s: %d elements differ from the exact result, first %s"
                             % (what, len(bad), bad[:5].tolist()))


class Guarded:
    """A device buffer of `shape` with canary regions on both sides."""

    def __init__(self, host_bits: np.ndarray, dtype: str, fill=None):
        import torch
        from gather_lora_matmul_amd.synthetic import to_device
        self.dtype = dtype
        self.shape = host_bits.shape
        flat = np.ascontiguousarray(host_bits).reshape(-1)
        canary = np.full(GUARD, 0x7A5A if dtype != "f32" else 12345.678,
                         np.uint16 if dtype != "f32" else np.float32)
        self.canary = canary
        full = np.concatenate([canary, flat, canary])
        self.buf = to_device(full, dtype)
        self.view = self.buf[GUARD:GUARD + flat.size].view(*self.shape) if flat.size else self.buf[GUARD:GUARD]
        del torch

    def host(self) -> np.ndarray:
        from gather_lora_matmul_amd.synthetic import from_device
        full = from_device(self.buf, self.dtype)
        lo, hi = full[:GUARD], full[-GUARD:]
        assert lo.tobytes() == self.canary.tobytes() and hi.tobytes() == self.canary.tobytes(), \
            "canary overwritten"
        return full[GUARD:-GUARD].reshape(self.shape)


def ids_tensor(ids: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()


def oracle_threads() -> int:
    import os
    return max(1, min(16, os.cpu_count() or 1))


def reference(wl, batch, s: int, y_dtype: str, subset: Optional[Sequence[int]] = None,
              threads: Optional[int] = None, return_v: bool = False):
    return oracle.workload_reference(wl, batch, s, y_dtype=y_dtype, token_subset=subset,
                                     n_threads=threads or oracle_threads(), return_v=return_v)


# ---------------------------------------------------------------------------
# running the HIP path through the C ABI on a workload batch
# ---------------------------------------------------------------------------
def run_bgmv(sp, batch, slices, y_dtype, mode, return_v=False):
    """mode: 'split' (shrink -> expand per slice) or 'fused' (one multi-slice apply).
    Returns {slice: y bits}, and with return_v also {slice: v} (split mode)."""
    import torch
    import gather_lora_matmul_amd as L
    from gather_lora_matmul_amd.synthetic import to_device
    wl = sp.wl
    ids = ids_tensor(batch.ids)
    n = len(batch.ids)
    xs = {s: to_device(batch.x[s], wl.act_dtype) for s in slices}
    ys = {s: Guarded(batch.y0[s], y_dtype) for s in slices}
    ydt = W.DTYPE_CODE[y_dtype]
    vs = {}
    if mode == "split":
        v_ld = sp.max_rank
        for s in slices:
            v = Guarded(np.full((n, v_ld), np.nan, np.float32), "f32")
            L.lora_bgmv_shrink(sp.handle, s, xs[s], ids, v.view, v_ld)
            L.lora_bgmv_expand(sp.handle, s, v.view, ids, ys[s].view, ydt, v_ld=v_ld)
            vs[s] = v
    else:
        L.lora_bgmv_apply(sp.handle, [(s, xs[s], ys[s].view) for s in slices], ids, ydt)
    torch.cuda.synchronize()
    out = {s: ys[s].host() for s in slices}
    vh = {s: v.host() for s, v in vs.items()}
    return (out, vh) if return_v else out


def run_sgmv(sp, batch, slices, y_dtype, mode, l_long=0, return_v=False):
    import torch
    import gather_lora_matmul_amd as L
    from gather_lora_matmul_amd.synthetic import prepare_shapes, to_device
    wl = sp.wl
    n = len(batch.ids)
    plan = L.lora_plan_create(sp.handle, max(1, n))
    L.lora_plan_build(plan, batch.ids, l_long=l_long)
    shapes = [[s] for s in slices] if mode == "split" else [list(slices)]
    ws = prepare_shapes(plan, shapes)
    xs = {s: to_device(batch.x[s], wl.act_dtype) for s in slices}
    ys = {s: Guarded(batch.y0[s], y_dtype) for s in slices}
    ydt = W.DTYPE_CODE[y_dtype]
    vs = {}
    if mode == "split":
        v_ld = sp.max_rank
        for s in slices:
            v = Guarded(np.full((n, v_ld), np.nan, np.float32), "f32")
            L.lora_sgmv_shrink(sp.handle, plan, s, xs[s], v.view, v_ld, workspace=ws)
            L.lora_sgmv_expand(sp.handle, plan, s, v.view, ys[s].view, ydt, v_ld=v_ld)
            vs[s] = v
    else:
        L.lora_apply(sp.handle, plan, [(s, xs[s], ys[s].view) for s in slices], ydt, workspace=ws)
    torch.cuda.synchronize()
    stats = L.lora_plan_get_stats(plan)
    L.lora_plan_destroy(plan)
    out = {s: ys[s].host() for s in slices}
    vh = {s: v.host() for s, v in vs.items()}
    return (out, stats, vh) if return_v else (out, stats)


def check_all(wl, b, ys, vs, slices, y_dtype, label):
    """Every row of every slice against the oracle; v too when the split calls
    produced it; the LoRA delta itself when y is fp32 on a non-zero y0."""
    for s in slices:
        if s in vs:
            y_ref, v_ref = reference(wl, b, s, y_dtype, return_v=True)
            compare_v(vs[s], v_ref, b.ids, wl.ranks, "%s s%d" % (label, s))
        else:
            y_ref = reference(wl, b, s, y_dtype)
        compare(ys[s], y_ref, y_dtype, "%s s%d" % (label, s), y0_bits=b.y0[s])



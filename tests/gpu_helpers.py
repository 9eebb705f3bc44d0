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


def compare(y_gpu_bits: np.ndarray, y_ref: np.ndarray, y_dtype: str, what: str = ""):
    """Gate A (fp32 y): against the unrounded fp64 result.  Gate B (16-bit y):
    against the oracle's result rounded once to the y dtype."""
    if y_dtype == "f32":
        cmp = y_ref
    else:
        cmp = oracle.decode(oracle.round_to(y_ref, y_dtype), y_dtype)
    g = W.dequantize(y_gpu_bits, y_dtype)
    assert g.shape == cmp.shape, (g.shape, cmp.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite output (poisoned page read?)" % what
    d = g - cmp
    nrm = np.linalg.norm(cmp)
    rel = np.linalg.norm(d) / nrm if nrm > 0 else np.linalg.norm(d)
    mx = np.abs(d).max() if d.size else 0.0
    bound = MAX_ABS * max(np.abs(y_ref).max() if y_ref.size else 0.0, 1e-30)
    assert rel <= REL_L2, "%s: rel L2 %.3e > %.1e" % (what, rel, REL_L2)
    assert mx <= bound, "%s: max abs %.3e > %.3e" % (what, mx, bound)
    return rel, mx


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


def reference(wl, batch, s: int, y_dtype: str, subset: Optional[Sequence[int]] = None,
              threads: int = 8):
    return oracle.workload_reference(wl, batch, s, y_dtype=y_dtype, token_subset=subset,
                                     n_threads=threads)

"""fp64 CPU oracle for y_i += s_a B_a (A_a x_i) -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import this package.  The HIP library never links or calls it, and it does
not import the HIP library: the two share nothing but the seeded input
generators in `workloads/`.

The arithmetic lives in `lora_oracle.c` (plain C, double precision, loops in
ascending index order).  This module compiles it with gcc and marshals numpy
arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblora_oracle.so")
_lib = None

DT = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}


def build(force: bool = True) -> str:
    """Compile the oracle (gcc, -O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    lib.oracle_round.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P]
    lib.oracle_decode.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P]
    lib.oracle_lora_apply.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, P, P, ctypes.c_int32, P, P, P, P, P, P, P, P, P, ctypes.c_int32,
        ctypes.c_int32]
    lib.oracle_walk_adapter.argtypes = [
        P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, P, P, P, P]
    lib.oracle_max_threads.argtypes = []
    for f in ("oracle_round", "oracle_decode", "oracle_lora_apply", "oracle_walk_adapter",
              "oracle_max_threads"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _storage(dtype: str):
    return {"f32": np.float32, "e4m3": np.uint8}.get(dtype, np.uint16)


def round_to(values: np.ndarray, dtype: str) -> np.ndarray:
    """RNE-round float64 values to `dtype` (f32, f16, bf16); returns the stored form."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.float32 if dtype == "f32" else np.uint16)
    rc = _load().oracle_round(_ptr(v), v.size, DT[dtype], _ptr(out))
    if rc:
        raise ValueError("oracle_round failed: %d" % rc)
    return out


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    b = np.ascontiguousarray(bits)
    out = np.empty(b.shape, np.float64)
    rc = _load().oracle_decode(_ptr(b), b.size, DT[dtype], _ptr(out))
    if rc:
        raise ValueError("oracle_decode failed: %d" % rc)
    return out


def lora_apply(x_bits: np.ndarray, ids: np.ndarray, ranks: np.ndarray, scales: np.ndarray,
               weights: Dict[int, tuple], y0_bits: np.ndarray,
               w_dtype: str, y_dtype: str, return_v: bool = False, v_ld: int = 0,
               n_threads: int = 1, x_dtype: Optional[str] = None):
    """y_ref (float64 [n][d_out]) of y_i = y0_i + s_a B_a (A_a x_i).

    `weights` maps adapter id -> (A bits [r][d_in], B bits [d_out][r]) or, for a
    quantised adapter, (A codes, B codes, a_scale [r], b_scale [r]); only the
    adapters that the batch names need to be present.  x is in x_dtype (default
    w_dtype)."""
    x_dtype = x_dtype or w_dtype
    x = np.ascontiguousarray(x_bits)
    y0 = np.ascontiguousarray(y0_bits)
    ids = np.ascontiguousarray(ids, np.int32)
    n, d_in = x.shape
    d_out = y0.shape[1]
    assert y0.shape[0] == n and ids.shape[0] == n
    ranks = np.ascontiguousarray(ranks, np.int32)
    scales = np.ascontiguousarray(scales, np.float32)
    na = ranks.shape[0]
    Ap = (ctypes.c_void_p * na)()
    Bp = (ctypes.c_void_p * na)()
    SAp = (ctypes.c_void_p * na)()
    SBp = (ctypes.c_void_p * na)()
    quant = False
    keep = []
    for a, wt in weights.items():
        A = np.ascontiguousarray(wt[0])
        B = np.ascontiguousarray(wt[1])
        r = int(ranks[a])
        assert A.shape == (r, d_in) and B.shape == (d_out, r), (a, A.shape, B.shape, r)
        keep += [A, B]
        Ap[a] = _ptr(A)
        Bp[a] = _ptr(B)
        if len(wt) == 4:
            sa = np.ascontiguousarray(wt[2], np.float32)
            sb = np.ascontiguousarray(wt[3], np.float32)
            assert sa.shape == (r,) and sb.shape == (r,)
            keep += [sa, sb]
            SAp[a] = _ptr(sa)
            SBp[a] = _ptr(sb)
            quant = True
    y = np.empty((n, d_out), np.float64)
    if return_v:
        v_ld = v_ld or int(ranks.max())
        v = np.empty((n, v_ld), np.float64)
        vp = _ptr(v)
    else:
        v, vp = None, None
    sa_arg = ctypes.cast(SAp, ctypes.c_void_p) if quant else None
    sb_arg = ctypes.cast(SBp, ctypes.c_void_p) if quant else None
    rc = _load().oracle_lora_apply(n, d_in, d_out, DT[w_dtype], DT[x_dtype], DT[y_dtype], _ptr(x),
                                   _ptr(ids), na, _ptr(ranks), _ptr(scales),
                                   ctypes.cast(Ap, ctypes.c_void_p), ctypes.cast(Bp, ctypes.c_void_p),
                                   sa_arg, sb_arg, _ptr(y0), _ptr(y), vp, v_ld, n_threads)
    if rc == -1:
        raise KeyError("a token names an adapter whose weights were not supplied")
    if rc:
        raise ValueError("oracle_lora_apply failed: %d" % rc)
    return (y, v) if return_v else y


def walk_adapter(pool_bits: np.ndarray, dtype: str, page_elems: int, d_in: int, d_out: int,
                 rank: int, a_pages: np.ndarray, b_pages: np.ndarray):
    """Rebuild dense (A, B) bits of one adapter slice from a host pool image."""
    pool = np.ascontiguousarray(pool_bits)
    n_pages = pool.size // page_elems
    sd = _storage(dtype)
    A = np.empty((rank, d_in), sd)
    B = np.empty((d_out, rank), sd)
    ap = np.ascontiguousarray(a_pages, np.int32)
    bp = np.ascontiguousarray(b_pages, np.int32)
    rc = _load().oracle_walk_adapter(_ptr(pool), DT[dtype], page_elems, n_pages, d_in, d_out,
                                     rank, _ptr(ap), _ptr(bp), _ptr(A), _ptr(B))
    if rc == -1:
        raise IndexError("page id out of range")
    if rc == -4:
        raise ValueError("non-zero padding column in a B page")
    if rc:
        raise ValueError("oracle_walk_adapter failed: %d" % rc)
    return A, B


def workload_reference(wl, batch, slice_idx: int, y_dtype: Optional[str] = None,
                       token_subset: Optional[Sequence[int]] = None, n_threads: int = 1,
                       return_v: bool = False):
    """Oracle result for one slice of a workload batch (optionally on a subset
    of tokens, for full-size sampled checks)."""
    y_dtype = y_dtype or wl.act_dtype
    x = batch.x[slice_idx]
    y0 = batch.y0[slice_idx]
    ids = batch.ids
    if token_subset is not None:
        sel = np.asarray(token_subset, np.int64)
        x, y0, ids = x[sel], y0[sel], ids[sel]
    used = sorted(set(int(a) for a in ids.tolist() if a >= 0))
    weights = {}
    for a in used:
        A, B = wl.weights(a, slice_idx)
        q = wl.qscales(a, slice_idx)
        weights[a] = (A, B) if q is None else (A, B, q[0], q[1])
    return lora_apply(x, ids, wl.ranks, wl.scales, weights, y0, wl.dtype, y_dtype,
                      return_v=return_v, v_ld=wl.max_rank if return_v else 0,
                      n_threads=n_threads, x_dtype=wl.act_dtype)

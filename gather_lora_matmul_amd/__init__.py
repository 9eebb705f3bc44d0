"""Python binding of liblora_mi355x.so (heterogeneous-adapter LoRA apply on MI355X).

Argument marshalling only: every function here forwards to the C entry point of
the same name in `include/lora_mi355x.h`; all arithmetic runs in the HIP kernels.
Tensors are passed as raw device pointers, the stream as the current torch
stream's hipStream_t.  There is no fallback: if the library is not built the
import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblora_mi355x.so")

LORA_F32, LORA_F16, LORA_BF16 = 0, 1, 2
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
LORA_OK = 0
STATUS = {0: "LORA_OK", -1: "LORA_E_ARG", -2: "LORA_E_NOMEM", -3: "LORA_E_NOT_RESIDENT",
          -4: "LORA_E_RANK", -5: "LORA_E_STATE", -6: "LORA_E_HIP", -7: "LORA_E_UNSUPPORTED"}
LORA_POOL_POISON = 1
LORA_POOL_HOST_ONLY = 2
LORA_MAX_SLICES = 16
LORA_MAX_RANK = 128
LORA_MAX_IO = 8

# Every symbol the header declares.
EXPORTS = (
    "lora_pool_create", "lora_pool_destroy", "lora_pool_info", "lora_pool_alloc_pages",
    "lora_pool_free_pages", "lora_pool_upload", "lora_pool_evict", "lora_page_table_build",
    "lora_pool_export_entry", "lora_pool_read_pages", "lora_bgmv_shrink", "lora_bgmv_expand",
    "lora_bgmv_apply", "lora_plan_create", "lora_plan_destroy", "lora_plan_build",
    "lora_plan_get_stats", "lora_plan_export", "lora_sgmv_shrink", "lora_sgmv_expand",
    "lora_apply", "lora_debug_resolve", "lora_debug_gather", "lora_last_error",
)


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status), msg))
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("page_elems", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_pages", ctypes.c_int64), ("max_adapters", ctypes.c_int32),
                ("max_rank", ctypes.c_int32), ("n_slices", ctypes.c_int32),
                ("slice_d_in", ctypes.POINTER(ctypes.c_int32)),
                ("slice_d_out", ctypes.POINTER(ctypes.c_int32)),
                ("shuffle_seed", ctypes.c_uint64), ("flags", ctypes.c_uint32),
                ("pages_dev", ctypes.c_void_p)]


class Io(ctypes.Structure):
    _fields_ = [("slice", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("x_dev", ctypes.c_void_p), ("y_dev", ctypes.c_void_p)]


class PlanStats(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("n_items", ctypes.c_int32), ("n_mfma_items", ctypes.c_int32),
                ("mfma_tokens", ctypes.c_int32), ("l_long", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblora_mi355x.so is not built: run `python gather_lora_matmul_amd/build.py`")
    # One HIP runtime per process: torch ships its own libamdhip64 (same soname
    # as ROCm's), and of two runtimes in one process only the first to start
    # sees the GPU.  With torch loaded first, this library binds to its runtime
    # and shares device pointers and streams with it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    V, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sig = {
        "lora_pool_create": [ctypes.POINTER(PoolDesc), ctypes.POINTER(V)],
        "lora_pool_destroy": [V],
        "lora_pool_info": [V, ctypes.POINTER(I64), ctypes.POINTER(V)],
        "lora_pool_alloc_pages": [V, I64, V],
        "lora_pool_free_pages": [V, I64, V],
        "lora_pool_upload": [V, I32, I32, I32, F, V, V, V],
        "lora_pool_evict": [V, I32, I32, V],
        "lora_page_table_build": [V, V],
        "lora_pool_export_entry": [V, I32, I32, V, V, V, V, V, V],
        "lora_pool_read_pages": [V, I64, I64, V],
        "lora_bgmv_shrink": [V, I32, V, V, I32, V, I32, V],
        "lora_bgmv_expand": [V, I32, V, I32, V, I32, V, V, I32, V],
        "lora_bgmv_apply": [V, I32, ctypes.POINTER(Io), V, I32, I32, V],
        "lora_plan_create": [V, I32, ctypes.POINTER(V)],
        "lora_plan_destroy": [V],
        "lora_plan_build": [V, V, I32, I32, V],
        "lora_plan_get_stats": [V, ctypes.POINTER(PlanStats)],
        "lora_plan_export": [V, V, V],
        "lora_sgmv_shrink": [V, V, I32, V, V, I32, V],
        "lora_sgmv_expand": [V, V, I32, V, I32, V, I32, V],
        "lora_apply": [V, V, I32, ctypes.POINTER(Io), I32, V],
        "lora_debug_resolve": [V, I32, V, I32, V, V, V],
        "lora_debug_gather": [V, I32, I32, V, V, V],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.lora_last_error.argtypes = []
    lib.lora_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int, where: str):
    if status != LORA_OK:
        raise LoraError(status, where, _lib.lora_last_error().decode(errors="replace"))


def _np_ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _dev_ptr(t) -> int:
    """Device pointer of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


# ----------------------------------------------------------------------------
# pool
# ----------------------------------------------------------------------------
def lora_pool_create(page_elems: int, dtype: int, n_pages: int, max_adapters: int, max_rank: int,
                     slice_dims: Sequence[Tuple[int, int]], shuffle_seed: int = 0, flags: int = 0,
                     pages_dev=None) -> int:
    """Returns an opaque pool handle (int).  `pages_dev` may be a torch tensor
    that provides the page memory (the caller keeps it alive)."""
    ns = len(slice_dims)
    din = (ctypes.c_int32 * ns)(*[int(a) for a, _ in slice_dims])
    dout = (ctypes.c_int32 * ns)(*[int(b) for _, b in slice_dims])
    d = PoolDesc(page_elems, dtype, n_pages, max_adapters, max_rank, ns, din, dout,
                 shuffle_seed, flags, _dev_ptr(pages_dev) if pages_dev is not None else None)
    h = ctypes.c_void_p()
    _check(_lib.lora_pool_create(ctypes.byref(d), ctypes.byref(h)), "lora_pool_create")
    return h.value


def lora_pool_destroy(pool: int):
    _check(_lib.lora_pool_destroy(pool), "lora_pool_destroy")


def lora_pool_info(pool: int) -> Tuple[int, int]:
    free = ctypes.c_int64()
    base = ctypes.c_void_p()
    _check(_lib.lora_pool_info(pool, ctypes.byref(free), ctypes.byref(base)), "lora_pool_info")
    return free.value, base.value


def lora_pool_alloc_pages(pool: int, n: int) -> np.ndarray:
    ids = np.empty(n, np.int32)
    _check(_lib.lora_pool_alloc_pages(pool, n, _np_ptr(ids) if n else None), "lora_pool_alloc_pages")
    return ids


def lora_pool_free_pages(pool: int, ids: np.ndarray):
    ids = np.ascontiguousarray(ids, np.int32)
    _check(_lib.lora_pool_free_pages(pool, ids.size, _np_ptr(ids) if ids.size else None),
           "lora_pool_free_pages")


def lora_pool_upload(pool: int, adapter: int, slice_: int, rank: int, scale: float,
                     A_host: np.ndarray, B_host: np.ndarray, stream=None):
    A = np.ascontiguousarray(A_host)
    B = np.ascontiguousarray(B_host)
    _check(_lib.lora_pool_upload(pool, adapter, slice_, rank, float(scale), _np_ptr(A), _np_ptr(B),
                                 stream if isinstance(stream, int) else None),
           "lora_pool_upload")


def lora_pool_evict(pool: int, adapter: int, slice_: int, stream=None):
    _check(_lib.lora_pool_evict(pool, adapter, slice_, stream if isinstance(stream, int) else None),
           "lora_pool_evict")


def lora_page_table_build(pool: int, stream=None):
    _check(_lib.lora_page_table_build(pool, stream if isinstance(stream, int) else None),
           "lora_page_table_build")


def lora_pool_export_entry(pool: int, adapter: int, slice_: int):
    """-> (rank, scale, a_pages, b_pages)"""
    r, na, nb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    sc = ctypes.c_float()
    _check(_lib.lora_pool_export_entry(pool, adapter, slice_, ctypes.byref(r), ctypes.byref(sc),
                                       ctypes.byref(na), None, ctypes.byref(nb), None),
           "lora_pool_export_entry")
    a = np.empty(na.value, np.int32)
    b = np.empty(nb.value, np.int32)
    _check(_lib.lora_pool_export_entry(pool, adapter, slice_, None, None, None,
                                       _np_ptr(a) if a.size else None, None,
                                       _np_ptr(b) if b.size else None),
           "lora_pool_export_entry")
    return r.value, sc.value, a, b


def lora_pool_read_pages(pool: int, first: int, count: int, page_elems: int, dtype: int) -> np.ndarray:
    out = np.empty(count * page_elems, np.float32 if dtype == LORA_F32 else np.uint16)
    _check(_lib.lora_pool_read_pages(pool, first, count, _np_ptr(out)), "lora_pool_read_pages")
    return out


# ----------------------------------------------------------------------------
# BGMV
# ----------------------------------------------------------------------------
def lora_bgmv_shrink(pool: int, slice_: int, x, ids, v, v_ld: Optional[int] = None, stream=None):
    n = int(ids.shape[0])
    v_ld = int(v.shape[1]) if v_ld is None else v_ld
    _check(_lib.lora_bgmv_shrink(pool, slice_, _dev_ptr(x), _dev_ptr(ids), n, _dev_ptr(v), v_ld,
                                 _stream(stream)), "lora_bgmv_shrink")


def lora_bgmv_expand(pool: int, slice_: int, v, ids, y, y_dtype: int, token_scale=None,
                     v_ld: Optional[int] = None, stream=None):
    n = int(ids.shape[0])
    v_ld = int(v.shape[1]) if v_ld is None else v_ld
    _check(_lib.lora_bgmv_expand(pool, slice_, _dev_ptr(v), v_ld, _dev_ptr(ids), n,
                                 _dev_ptr(token_scale), _dev_ptr(y), y_dtype, _stream(stream)),
           "lora_bgmv_expand")


def _ios(ios: Sequence[Tuple[int, object, object]]):
    arr = (Io * len(ios))()
    for k, (s, x, y) in enumerate(ios):
        arr[k] = Io(int(s), 0, _dev_ptr(x), _dev_ptr(y))
    return arr


def lora_bgmv_apply(pool: int, ios: Sequence[Tuple[int, object, object]], ids, y_dtype: int,
                    stream=None):
    """ios: [(slice, x, y), ...] sharing `ids`."""
    arr = _ios(ios)
    _check(_lib.lora_bgmv_apply(pool, len(ios), arr, _dev_ptr(ids), int(ids.shape[0]), y_dtype,
                                _stream(stream)), "lora_bgmv_apply")


# ----------------------------------------------------------------------------
# SGMV
# ----------------------------------------------------------------------------
def lora_plan_create(pool: int, max_tokens: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib.lora_plan_create(pool, max_tokens, ctypes.byref(h)), "lora_plan_create")
    return h.value


def lora_plan_destroy(plan: int):
    _check(_lib.lora_plan_destroy(plan), "lora_plan_destroy")


def lora_plan_build(plan: int, ids_host: np.ndarray, l_long: int = 0, stream=None):
    ids = np.ascontiguousarray(ids_host, np.int32)
    st = stream if isinstance(stream, int) else (_stream(stream) if stream is not None else None)
    if st is None:
        try:
            st = _stream(None)
        except Exception:
            st = None
    _check(_lib.lora_plan_build(plan, _np_ptr(ids) if ids.size else None, ids.size, l_long, st),
           "lora_plan_build")


def lora_plan_get_stats(plan: int) -> dict:
    s = PlanStats()
    _check(_lib.lora_plan_get_stats(plan, ctypes.byref(s)), "lora_plan_get_stats")
    return {f: getattr(s, f) for f, _ in PlanStats._fields_}


def lora_plan_export(plan: int) -> Tuple[np.ndarray, np.ndarray]:
    st = lora_plan_get_stats(plan)
    perm = np.empty(st["n_tokens"], np.int32)
    items = np.empty((st["n_items"], 4), np.int32)
    _check(_lib.lora_plan_export(plan, _np_ptr(perm) if perm.size else None,
                                 _np_ptr(items) if items.size else None), "lora_plan_export")
    return perm, items


def lora_sgmv_shrink(pool: int, plan: int, slice_: int, x, v, v_ld: Optional[int] = None,
                     stream=None):
    v_ld = int(v.shape[1]) if v_ld is None else v_ld
    _check(_lib.lora_sgmv_shrink(pool, plan, slice_, _dev_ptr(x), _dev_ptr(v), v_ld,
                                 _stream(stream)), "lora_sgmv_shrink")


def lora_sgmv_expand(pool: int, plan: int, slice_: int, v, y, y_dtype: int,
                     v_ld: Optional[int] = None, stream=None):
    v_ld = int(v.shape[1]) if v_ld is None else v_ld
    _check(_lib.lora_sgmv_expand(pool, plan, slice_, _dev_ptr(v), v_ld, _dev_ptr(y), y_dtype,
                                 _stream(stream)), "lora_sgmv_expand")


def lora_apply(pool: int, plan: int, ios: Sequence[Tuple[int, object, object]], y_dtype: int,
               stream=None):
    arr = _ios(ios)
    _check(_lib.lora_apply(pool, plan, len(ios), arr, y_dtype, _stream(stream)), "lora_apply")


# ----------------------------------------------------------------------------
# verification
# ----------------------------------------------------------------------------
def lora_debug_resolve(pool: int, slice_: int, ids, a_off, b_off, stream=None):
    _check(_lib.lora_debug_resolve(pool, slice_, _dev_ptr(ids), int(ids.shape[0]), _dev_ptr(a_off),
                                   _dev_ptr(b_off), _stream(stream)), "lora_debug_resolve")


def lora_debug_gather(pool: int, slice_: int, adapter: int, A, B, stream=None):
    _check(_lib.lora_debug_gather(pool, slice_, adapter, _dev_ptr(A), _dev_ptr(B), _stream(stream)),
           "lora_debug_gather")


def lora_last_error() -> str:
    return _lib.lora_last_error().decode(errors="replace")

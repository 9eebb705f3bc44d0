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
# LORA_MI355X_LIB: another build of the library (the profiling build)
LIB_PATH = os.environ.get("LORA_MI355X_LIB") or os.path.join(_HERE, "liblora_mi355x.so")

LORA_F32, LORA_F16, LORA_BF16, LORA_FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
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
    "lora_pool_free_pages", "lora_pool_upload", "lora_pool_upload_scaled", "lora_pool_evict",
    "lora_page_table_build", "lora_pool_export_entry", "lora_pool_export_scales",
    "lora_pool_read_pages", "lora_bgmv_shrink", "lora_bgmv_expand",
    "lora_bgmv_apply", "lora_bgmv_planned_workspace_size", "lora_bgmv_apply_planned",
    "lora_dplan_create", "lora_dplan_destroy", "lora_dplan_build", "lora_dplan_apply",
    "lora_plan_create", "lora_plan_destroy", "lora_plan_build",
    "lora_plan_get_stats", "lora_plan_export", "lora_plan_prepare", "lora_workspace_size",
    "lora_sgmv_shrink", "lora_sgmv_expand", "lora_apply", "lora_apply_noalloc", "lora_debug_resolve",
    "lora_debug_gather", "lora_debug_decode", "lora_debug_block_timeline", "lora_last_error",
    "lora_store_create",
    "lora_store_destroy", "lora_store_add", "lora_store_ensure", "lora_store_get_stats",
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
                ("pages_dev", ctypes.c_void_p), ("act_dtype", ctypes.c_int32)]


class Io(ctypes.Structure):
    _fields_ = [("slice", ctypes.c_int32), ("x_group", ctypes.c_int32),
                ("x_dev", ctypes.c_void_p), ("y_dev", ctypes.c_void_p)]


class StoreStats(ctypes.Structure):
    _fields_ = [("uploads", ctypes.c_int64), ("evictions", ctypes.c_int64),
                ("bytes_uploaded", ctypes.c_int64), ("resident", ctypes.c_int32),
                ("registered", ctypes.c_int32)]


class PlanStats(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("n_items", ctypes.c_int32), ("n_mfma_items", ctypes.c_int32),
                ("mfma_tokens", ctypes.c_int32), ("l_long", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("%s is not built: run `python gather_lora_matmul_amd/build.py`" % LIB_PATH)
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
        "lora_pool_upload_scaled": [V, I32, I32, I32, F, V, V, V, V, V],
        "lora_pool_export_scales": [V, I32, I32, V, V],
        "lora_debug_decode": [I32, V, I64, V, V],
        "lora_debug_block_timeline": [V, ctypes.c_size_t],
        "lora_store_create": [V, ctypes.POINTER(V)],
        "lora_store_destroy": [V],
        "lora_store_add": [V, I32, I32, I32, F, V, V, V, V],
        "lora_store_ensure": [V, I32, V, V, V],
        "lora_store_get_stats": [V, ctypes.POINTER(StoreStats)],
        "lora_pool_evict": [V, I32, I32, V],
        "lora_page_table_build": [V, V],
        "lora_pool_export_entry": [V, I32, I32, V, V, V, V, V, V],
        "lora_pool_read_pages": [V, I64, I64, V],
        "lora_bgmv_shrink": [V, I32, V, V, I32, V, I32, V],
        "lora_bgmv_expand": [V, I32, V, I32, V, I32, V, V, I32, V],
        "lora_bgmv_apply": [V, I32, ctypes.POINTER(Io), V, I32, I32, V],
        "lora_bgmv_planned_workspace_size": [V, I32, ctypes.POINTER(Io), I32,
                                             ctypes.POINTER(ctypes.c_size_t)],
        "lora_bgmv_apply_planned": [V, I32, ctypes.POINTER(Io), V, I32, I32, V, ctypes.c_size_t, V],
        "lora_dplan_create": [V, I32, I32, ctypes.POINTER(Io), ctypes.POINTER(V)],
        "lora_dplan_destroy": [V],
        "lora_dplan_build": [V, I32, ctypes.POINTER(Io), V, I32, V],
        "lora_dplan_apply": [V, V, I32, ctypes.POINTER(Io), I32, V],
        "lora_plan_create": [V, I32, ctypes.POINTER(V)],
        "lora_plan_destroy": [V],
        "lora_plan_build": [V, V, I32, I32, V],
        "lora_plan_get_stats": [V, ctypes.POINTER(PlanStats)],
        "lora_plan_export": [V, V, V],
        "lora_plan_prepare": [V, I32, ctypes.POINTER(Io), V],
        "lora_workspace_size": [V, I32, ctypes.POINTER(Io), ctypes.POINTER(ctypes.c_size_t)],
        "lora_sgmv_shrink": [V, V, I32, V, V, I32, V, ctypes.c_size_t, V],
        "lora_sgmv_expand": [V, V, I32, V, I32, V, I32, V],
        "lora_apply": [V, V, I32, ctypes.POINTER(Io), I32, V, ctypes.c_size_t, V],
        "lora_apply_noalloc": [V, V, I32, ctypes.POINTER(Io), I32, V],
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


# Shapes of the pools created through this binding (handle -> (dtype, slice
# dims, max_rank)), so that buffers can be checked before a call: the C ABI
# takes raw pointers and cannot see their sizes or element types.
_POOLS = {}
_PLAN_POOL = {}
_DT_NAME = {0: "float32", 1: "float16", 2: "bfloat16"}


def _check_tensor(t, what: str, dtype_code: Optional[int], min_numel: int):
    import torch
    if t is None:
        raise ValueError("%s: missing tensor" % what)
    if dtype_code is not None and t.dtype != getattr(torch, _DT_NAME[dtype_code]):
        raise TypeError("%s: dtype %s, expected %s" % (what, t.dtype, _DT_NAME[dtype_code]))
    if t.numel() < min_numel:
        raise ValueError("%s: %d elements, the call reads or writes %d" % (what, t.numel(), min_numel))


def _check_ids(ids):
    import torch
    if ids.dtype != torch.int32 or ids.dim() != 1:
        raise TypeError("ids: expected a 1-D int32 tensor, got %s %s" % (ids.dtype, tuple(ids.shape)))


def _check_io(pool: int, ios, n: int, y_dtype: int):
    info = _POOLS.get(pool)
    for k, e in enumerate(ios):
        s, x, y = e[:3]
        if info is None:
            continue
        dt, dims, _ = info
        if not 0 <= int(s) < len(dims):
            continue  # the library reports the bad slice
        d_in, d_out = dims[int(s)]
        _check_tensor(x, "io %d x" % k, dt, n * d_in)
        _check_tensor(y, "io %d y" % k, y_dtype, n * d_out)


def _check_v(pool: int, v, n: int, v_ld: int):
    _check_tensor(v, "v", 0, n * v_ld)


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
                     pages_dev=None, act_dtype: Optional[int] = None) -> int:
    """Returns an opaque pool handle (int).  `pages_dev` may be a torch tensor
    that provides the page memory (the caller keeps it alive).  act_dtype: the
    dtype of x (default: the page dtype; f16 or bf16 for FP8 pages)."""
    ns = len(slice_dims)
    din = (ctypes.c_int32 * ns)(*[int(a) for a, _ in slice_dims])
    dout = (ctypes.c_int32 * ns)(*[int(b) for _, b in slice_dims])
    act = dtype if act_dtype is None else act_dtype
    d = PoolDesc(page_elems, dtype, n_pages, max_adapters, max_rank, ns, din, dout,
                 shuffle_seed, flags, _dev_ptr(pages_dev) if pages_dev is not None else None, act)
    h = ctypes.c_void_p()
    _check(_lib.lora_pool_create(ctypes.byref(d), ctypes.byref(h)), "lora_pool_create")
    _POOLS[h.value] = (int(act), [(int(a), int(b)) for a, b in slice_dims], int(max_rank))
    return h.value


def lora_pool_destroy(pool: int):
    _POOLS.pop(pool, None)
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


def lora_pool_upload_scaled(pool: int, adapter: int, slice_: int, rank: int, scale: float,
                            A_host: np.ndarray, a_scale: np.ndarray, B_host: np.ndarray,
                            b_scale: np.ndarray, stream=None):
    A = np.ascontiguousarray(A_host)
    B = np.ascontiguousarray(B_host)
    sa = np.ascontiguousarray(a_scale, np.float32)
    sb = np.ascontiguousarray(b_scale, np.float32)
    if sa.size < rank or sb.size < rank:
        raise ValueError("scale arrays need rank entries")
    _check(_lib.lora_pool_upload_scaled(pool, adapter, slice_, rank, float(scale), _np_ptr(A),
                                        _np_ptr(sa), _np_ptr(B), _np_ptr(sb),
                                        stream if isinstance(stream, int) else None),
           "lora_pool_upload_scaled")


def lora_pool_export_scales(pool: int, adapter: int, slice_: int, rank: int):
    """-> (a_scale, b_scale) float32 [rank] of a quantised adapter slice."""
    sa = np.empty(rank, np.float32)
    sb = np.empty(rank, np.float32)
    _check(_lib.lora_pool_export_scales(pool, adapter, slice_, _np_ptr(sa), _np_ptr(sb)),
           "lora_pool_export_scales")
    return sa, sb


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
    out = np.empty(count * page_elems, {LORA_F32: np.float32, LORA_FP8_E4M3: np.uint8}.get(dtype, np.uint16))
    _check(_lib.lora_pool_read_pages(pool, first, count, _np_ptr(out)), "lora_pool_read_pages")
    return out


# ----------------------------------------------------------------------------
# host adapter store
# ----------------------------------------------------------------------------
def lora_store_create(pool: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib.lora_store_create(pool, ctypes.byref(h)), "lora_store_create")
    return h.value


def lora_store_destroy(store: int):
    _check(_lib.lora_store_destroy(store), "lora_store_destroy")


def lora_store_add(store: int, adapter: int, slice_: int, rank: int, scale: float,
                   A_host: np.ndarray, B_host: np.ndarray, a_scale=None, b_scale=None):
    A = np.ascontiguousarray(A_host)
    B = np.ascontiguousarray(B_host)
    sa = None if a_scale is None else np.ascontiguousarray(a_scale, np.float32)
    sb = None if b_scale is None else np.ascontiguousarray(b_scale, np.float32)
    _check(_lib.lora_store_add(store, adapter, slice_, rank, float(scale), _np_ptr(A),
                               None if sa is None else _np_ptr(sa), _np_ptr(B),
                               None if sb is None else _np_ptr(sb)), "lora_store_add")


def lora_store_ensure(store: int, adapters: np.ndarray, upload_stream=None, compute_stream=None):
    """upload_stream / compute_stream: raw hipStream_t ints or torch streams
    (None: torch's current stream)."""
    ids = np.ascontiguousarray(adapters, np.int32)
    up = upload_stream if isinstance(upload_stream, int) else _stream(upload_stream)
    cs = compute_stream if isinstance(compute_stream, int) else _stream(compute_stream)
    _check(_lib.lora_store_ensure(store, ids.size, _np_ptr(ids) if ids.size else None, up, cs),
           "lora_store_ensure")


def lora_store_get_stats(store: int) -> dict:
    st = StoreStats()
    _check(_lib.lora_store_get_stats(store, ctypes.byref(st)), "lora_store_get_stats")
    return {f: getattr(st, f) for f, _ in StoreStats._fields_}


# ----------------------------------------------------------------------------
# BGMV
# ----------------------------------------------------------------------------
def lora_bgmv_shrink(pool: int, slice_: int, x, ids, v, v_ld: Optional[int] = None, stream=None):
    _check_ids(ids)
    n = int(ids.shape[0])
    v_ld = int(v.shape[1]) if v_ld is None else v_ld
    info = _POOLS.get(pool)
    if info is not None and 0 <= slice_ < len(info[1]):
        _check_tensor(x, "x", info[0], n * info[1][slice_][0])
    _check_v(pool, v, n, v_ld)
    _check(_lib.lora_bgmv_shrink(pool, slice_, _dev_ptr(x), _dev_ptr(ids), n, _dev_ptr(v), v_ld,
                                 _stream(stream)), "lora_bgmv_shrink")


def lora_bgmv_expand(pool: int, slice_: int, v, ids, y, y_dtype: int, token_scale=None,
                     v_ld: Optional[int] = None, stream=None):
    _check_ids(ids)
    n = int(ids.shape[0])
    v_ld = int(v.shape[1]) if v_ld is None else v_ld
    info = _POOLS.get(pool)
    if info is not None and 0 <= slice_ < len(info[1]):
        _check_tensor(y, "y", y_dtype, n * info[1][slice_][1])
    _check_v(pool, v, n, v_ld)
    if token_scale is not None:
        _check_tensor(token_scale, "token_scale", 0, n)
    _check(_lib.lora_bgmv_expand(pool, slice_, _dev_ptr(v), v_ld, _dev_ptr(ids), n,
                                 _dev_ptr(token_scale), _dev_ptr(y), y_dtype, _stream(stream)),
           "lora_bgmv_expand")


def _ios(ios):
    """io entries (slice, x, y) or (slice, x, y, x_group) -> lora_io array."""
    arr = (Io * len(ios))()
    for k, e in enumerate(ios):
        s, x, y = e[:3]
        arr[k] = Io(int(s), int(e[3]) if len(e) > 3 else 0, _dev_ptr(x), _dev_ptr(y))
    return arr


def lora_bgmv_apply(pool: int, ios: Sequence[Tuple[int, object, object]], ids, y_dtype: int,
                    stream=None):
    """ios: [(slice, x, y) or (slice, x, y, x_group), ...] sharing `ids`."""
    _check_ids(ids)
    _check_io(pool, ios, int(ids.shape[0]), y_dtype)
    arr = _ios(ios)
    _check(_lib.lora_bgmv_apply(pool, len(ios), arr, _dev_ptr(ids), int(ids.shape[0]), y_dtype,
                                _stream(stream)), "lora_bgmv_apply")


def lora_bgmv_planned_workspace_size(pool: int, slices: Sequence[int], n: int) -> int:
    """Workspace bytes of lora_bgmv_apply_planned for n tokens over `slices`."""
    arr = _slice_ios(slices)
    out = ctypes.c_size_t()
    _check(_lib.lora_bgmv_planned_workspace_size(pool, len(slices), arr, int(n), ctypes.byref(out)),
           "lora_bgmv_planned_workspace_size")
    return int(out.value)


def lora_bgmv_apply_planned(pool: int, ios: Sequence[Tuple[int, object, object]], ids, y_dtype: int,
                            workspace, stream=None):
    """lora_bgmv_apply with the tokens grouped by adapter on the device (ids on
    the device); workspace: a device tensor of lora_bgmv_planned_workspace_size
    bytes, 256-byte aligned (torch's allocations are)."""
    _check_ids(ids)
    _check_io(pool, ios, int(ids.shape[0]), y_dtype)
    arr = _ios(ios)
    wp, wb = _ws(workspace)
    _check(_lib.lora_bgmv_apply_planned(pool, len(ios), arr, _dev_ptr(ids), int(ids.shape[0]), y_dtype,
                                        wp, wb, _stream(stream)), "lora_bgmv_apply_planned")


def lora_dplan_create(pool: int, max_tokens: int, slices: Sequence[int]) -> int:
    """A device plan for up to max_tokens tokens over slices of these shapes."""
    arr = _slice_ios(slices)
    h = ctypes.c_void_p()
    _check(_lib.lora_dplan_create(pool, int(max_tokens), len(slices), arr, ctypes.byref(h)),
           "lora_dplan_create")
    return h.value


def lora_dplan_destroy(dplan: int):
    _check(_lib.lora_dplan_destroy(dplan), "lora_dplan_destroy")


def lora_dplan_build(dplan: int, slices: Sequence[int], ids, stream=None):
    """Group the device ids by adapter (residency of `slices`) into the plan."""
    _check_ids(ids)
    arr = _slice_ios(slices)
    _check(_lib.lora_dplan_build(dplan, len(slices), arr, _dev_ptr(ids), int(ids.shape[0]),
                                 _stream(stream)), "lora_dplan_build")


def lora_dplan_apply(pool: int, dplan: int, ios: Sequence[Tuple[int, object, object]], n: int,
                     y_dtype: int, stream=None):
    """The plan's MFMA launches on ios (slices of the plan's shapes); n: the
    tokens of the last build (checks the x and y buffers)."""
    _check_io(pool, ios, int(n), y_dtype)
    arr = _ios(ios)
    _check(_lib.lora_dplan_apply(pool, dplan, len(ios), arr, y_dtype, _stream(stream)),
           "lora_dplan_apply")


# ----------------------------------------------------------------------------
# SGMV
# ----------------------------------------------------------------------------
def lora_plan_create(pool: int, max_tokens: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib.lora_plan_create(pool, max_tokens, ctypes.byref(h)), "lora_plan_create")
    _PLAN_POOL[h.value] = pool
    return h.value


def lora_plan_destroy(plan: int):
    _PLAN_POOL.pop(plan, None)
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


def _slice_ios(slices: Sequence[int]):
    arr = (Io * len(slices))()
    for k, s in enumerate(slices):
        arr[k] = Io(int(s), 0, None, None)
    return arr


def lora_plan_prepare(plan: int, slices: Sequence[int], stream=None):
    """Prepare the launch shape `slices` (the slices of a planned call, in order)."""
    arr = _slice_ios(slices)
    _check(_lib.lora_plan_prepare(plan, len(slices), arr, _stream(stream)), "lora_plan_prepare")


def lora_workspace_size(plan: int, slices: Sequence[int]) -> int:
    arr = _slice_ios(slices)
    out = ctypes.c_size_t()
    _check(_lib.lora_workspace_size(plan, len(slices), arr, ctypes.byref(out)),
           "lora_workspace_size")
    return int(out.value)


def _ws(workspace):
    """(pointer, bytes) of a caller-owned device workspace tensor (or None)."""
    if workspace is None:
        return None, 0
    return _dev_ptr(workspace), int(workspace.numel() * workspace.element_size())


def _plan_tokens(plan: int) -> int:
    return lora_plan_get_stats(plan)["n_tokens"]


def lora_sgmv_shrink(pool: int, plan: int, slice_: int, x, v, v_ld: Optional[int] = None,
                     workspace=None, stream=None):
    v_ld = int(v.shape[1]) if v_ld is None else v_ld
    n = _plan_tokens(plan)
    info = _POOLS.get(pool)
    if info is not None and 0 <= slice_ < len(info[1]):
        _check_tensor(x, "x", info[0], n * info[1][slice_][0])
    _check_v(pool, v, n, v_ld)
    wp, wb = _ws(workspace)
    _check(_lib.lora_sgmv_shrink(pool, plan, slice_, _dev_ptr(x), _dev_ptr(v), v_ld, wp, wb,
                                 _stream(stream)), "lora_sgmv_shrink")


def lora_sgmv_expand(pool: int, plan: int, slice_: int, v, y, y_dtype: int,
                     v_ld: Optional[int] = None, stream=None):
    v_ld = int(v.shape[1]) if v_ld is None else v_ld
    n = _plan_tokens(plan)
    info = _POOLS.get(pool)
    if info is not None and 0 <= slice_ < len(info[1]):
        _check_tensor(y, "y", y_dtype, n * info[1][slice_][1])
    _check_v(pool, v, n, v_ld)
    _check(_lib.lora_sgmv_expand(pool, plan, slice_, _dev_ptr(v), v_ld, _dev_ptr(y), y_dtype,
                                 _stream(stream)), "lora_sgmv_expand")


def lora_apply(pool: int, plan: int, ios: Sequence[Tuple[int, object, object]], y_dtype: int,
               workspace=None, stream=None):
    _check_io(pool, ios, _plan_tokens(plan), y_dtype)
    arr = _ios(ios)
    wp, wb = _ws(workspace)
    _check(_lib.lora_apply(pool, plan, len(ios), arr, y_dtype, wp, wb, _stream(stream)),
           "lora_apply")


def lora_apply_noalloc(pool: int, plan: int, ios: Sequence[Tuple[int, object, object]],
                       y_dtype: int, stream=None):
    """lora_apply with the library's static scratch as the workspace."""
    _check_io(pool, ios, _plan_tokens(plan), y_dtype)
    arr = _ios(ios)
    _check(_lib.lora_apply_noalloc(pool, plan, len(ios), arr, y_dtype, _stream(stream)),
           "lora_apply_noalloc")


# ----------------------------------------------------------------------------
# prepared calls: arguments checked and marshalled once
# ----------------------------------------------------------------------------
class PreparedCall:
    """A compute call whose buffers were checked and whose ctypes arguments were
    built once; calling it only invokes the C entry point on `stream` (a raw
    hipStream_t int, a torch stream, or None for torch's current stream).  The
    tensors it was made from must stay alive and keep their storage."""

    __slots__ = ("_fn", "_args", "_where", "_keep")

    def __init__(self, fn, args, where, keep):
        self._fn, self._args, self._where, self._keep = fn, tuple(args), where, keep

    def __call__(self, stream=None):
        st = self._fn(*self._args, stream if isinstance(stream, int) else _stream(stream))
        if st != LORA_OK:
            _check(st, self._where)


def prepare_bgmv_apply(pool: int, ios: Sequence[Tuple[int, object, object]], ids,
                       y_dtype: int) -> PreparedCall:
    _check_ids(ids)
    _check_io(pool, ios, int(ids.shape[0]), y_dtype)
    arr = _ios(ios)
    return PreparedCall(_lib.lora_bgmv_apply, (pool, len(ios), arr, _dev_ptr(ids),
                                               int(ids.shape[0]), y_dtype),
                        "lora_bgmv_apply", (ios, ids, arr))


def prepare_bgmv_apply_planned(pool: int, ios: Sequence[Tuple[int, object, object]], ids,
                               y_dtype: int, workspace) -> PreparedCall:
    _check_ids(ids)
    _check_io(pool, ios, int(ids.shape[0]), y_dtype)
    arr = _ios(ios)
    wp, wb = _ws(workspace)
    return PreparedCall(_lib.lora_bgmv_apply_planned, (pool, len(ios), arr, _dev_ptr(ids),
                                                       int(ids.shape[0]), y_dtype, wp, wb),
                        "lora_bgmv_apply_planned", (ios, ids, arr, workspace))


def prepare_dplan_apply(pool: int, dplan: int, ios: Sequence[Tuple[int, object, object]], n: int,
                        y_dtype: int) -> PreparedCall:
    _check_io(pool, ios, int(n), y_dtype)
    arr = _ios(ios)
    return PreparedCall(_lib.lora_dplan_apply, (pool, dplan, len(ios), arr, y_dtype),
                        "lora_dplan_apply", (ios, arr))


def prepare_apply(pool: int, plan: int, ios: Sequence[Tuple[int, object, object]], y_dtype: int,
                  workspace=None) -> PreparedCall:
    _check_io(pool, ios, _plan_tokens(plan), y_dtype)
    arr = _ios(ios)
    wp, wb = _ws(workspace)
    return PreparedCall(_lib.lora_apply, (pool, plan, len(ios), arr, y_dtype, wp, wb),
                        "lora_apply", (ios, workspace, arr))


# ----------------------------------------------------------------------------
# verification
# ----------------------------------------------------------------------------
def lora_debug_resolve(pool: int, slice_: int, ids, a_off, b_off, stream=None):
    _check(_lib.lora_debug_resolve(pool, slice_, _dev_ptr(ids), int(ids.shape[0]), _dev_ptr(a_off),
                                   _dev_ptr(b_off), _stream(stream)), "lora_debug_resolve")


def lora_debug_gather(pool: int, slice_: int, adapter: int, A, B, stream=None):
    _check(_lib.lora_debug_gather(pool, slice_, adapter, _dev_ptr(A), _dev_ptr(B), _stream(stream)),
           "lora_debug_gather")


def lora_debug_decode(dtype: int, src, dst, stream=None):
    """dst (float32) = the stored elements of src decoded by the kernels' decoder."""
    n = src.numel() * src.element_size() // {LORA_F32: 4, LORA_FP8_E4M3: 1}.get(dtype, 2)
    _check_tensor(dst, "dst", LORA_F32, n)
    _check(_lib.lora_debug_decode(dtype, _dev_ptr(src), n, _dev_ptr(dst), _stream(stream)),
           "lora_debug_decode")


def lora_debug_block_timeline(max_blocks: int) -> np.ndarray:
    """Per-block records [max_blocks][8] (uint64) of the last fused decode
    launch; raises LoraError(LORA_E_UNSUPPORTED) unless the library was built
    with `build.py --timeline` (and loaded through LORA_MI355X_LIB)."""
    out = np.zeros((max_blocks, 8), np.uint64)
    _check(_lib.lora_debug_block_timeline(out.ctypes.data, out.nbytes), "lora_debug_block_timeline")
    return out


def lora_last_error() -> str:
    return _lib.lora_last_error().decode(errors="replace")

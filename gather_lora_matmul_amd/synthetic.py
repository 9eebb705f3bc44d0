"""Populate a unified page pool from a synthetic workload (tests, bench, smoke).

Marshalling only: uploads the workload's adapters through `lora_pool_upload`,
interleaves KV-sized dummy pages through `lora_pool_alloc_pages`, and converts
between stored bit patterns (numpy) and device tensors (torch).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from . import (LORA_POOL_HOST_ONLY, LORA_POOL_POISON, DTYPE_CODE, lora_page_table_build,
               lora_plan_prepare, lora_pool_alloc_pages, lora_pool_create, lora_pool_destroy,
               lora_pool_upload, lora_pool_upload_scaled, lora_workspace_size)

_TORCH_DT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}
_ELT = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}


def torch_dtype(dtype: str):
    import torch
    return getattr(torch, _TORCH_DT[dtype])


def to_device(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    a = np.ascontiguousarray(bits)
    if dtype == "f32":
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    elif dtype == "e4m3":
        t = torch.from_numpy(a.view(np.uint8))
    else:
        t = torch.from_numpy(a.view(np.int16)).view(torch_dtype(dtype))
    return t.to(device)


def from_device(t, dtype: str) -> np.ndarray:
    import torch
    c = t.detach().contiguous().cpu()
    if dtype == "f32":
        return c.to(torch.float32).numpy()
    if dtype == "e4m3":
        return c.view(torch.uint8).numpy()
    return c.view(torch.int16).numpy().view(np.uint16)


def prepare_shapes(plan: int, shapes, stream=None):
    """Prepare the launch shapes (lists of slices) of a built plan and allocate
    one device workspace large enough for all of them (torch uint8, or None if
    none needs any).  Returns the workspace."""
    import torch
    need = 0
    for sl in shapes:
        lora_plan_prepare(plan, list(sl), stream=stream)
        need = max(need, lora_workspace_size(plan, list(sl)))
    if need == 0:
        return None
    return torch.empty(need, dtype=torch.uint8, device="cuda")


class SyntheticPool:
    """A pool holding (a subset of) a workload's adapters."""

    def __init__(self, wl, adapters: Optional[Iterable[int]] = None, host_only: bool = False,
                 poison: bool = True, n_pages: Optional[int] = None, max_rank: Optional[int] = None,
                 kv_dummy: Optional[float] = None):
        self.wl = wl
        self.dtype = wl.dtype
        self.dt = DTYPE_CODE[wl.dtype]
        self.P = wl.page_elems
        adapters = list(range(wl.n_adapters)) if adapters is None else sorted(set(adapters))
        self.adapters = adapters
        ratio = wl.kv_dummy_ratio if kv_dummy is None else kv_dummy
        if n_pages is None:
            # exact page count of the uploaded subset
            per16 = 16 // _ELT[wl.dtype]
            need = 0
            for a in adapters:
                r = int(wl.ranks[a])
                rs = -(-r // per16) * per16
                for d_in, d_out in wl.slices:
                    need += r * -(-d_in // self.P) + -(-d_out // (self.P // rs))
            n_pages = int(math.ceil(need * (wl.pool_slack + ratio))) + 8
        self.n_pages = n_pages
        self.max_rank = max_rank or wl.max_rank
        flags = (LORA_POOL_POISON if poison else 0) | (LORA_POOL_HOST_ONLY if host_only else 0)
        self.act = DTYPE_CODE[wl.act_dtype]
        self.handle = lora_pool_create(self.P, self.dt, n_pages, wl.n_adapters, self.max_rank,
                                       wl.slices, shuffle_seed=wl.shuffle_seed, flags=flags,
                                       act_dtype=self.act)
        self.kv_pages = []
        carry = 0.0
        for a in adapters:
            used = 0
            for s in range(len(wl.slices)):
                A, B = wl.weights(a, s)
                r = int(wl.ranks[a])
                q = wl.qscales(a, s)
                if q is None:
                    lora_pool_upload(self.handle, a, s, r, float(wl.scales[a]), A, B)
                else:
                    lora_pool_upload_scaled(self.handle, a, s, r, float(wl.scales[a]), A, q[0], B,
                                            q[1])
                d_in, d_out = wl.slices[s]
                per16 = 16 // _ELT[wl.dtype]
                rs = -(-r // per16) * per16
                used += r * -(-d_in // self.P) + -(-d_out // (self.P // rs))
            if ratio > 0:
                carry += ratio * used
                k = int(carry)
                carry -= k
                if k:
                    self.kv_pages.append(lora_pool_alloc_pages(self.handle, k))
        lora_page_table_build(self.handle)

    def close(self):
        if self.handle:
            lora_pool_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

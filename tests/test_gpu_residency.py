"""GPU tests of on-demand residency (host adapter store, loads on an upload
stream overlapping compute, LRU eviction, double-buffered page table) against
the fp64 oracle, through the C ABI.

The decisive case: each batch's adapters are disjoint from the previous
batch's and the pool holds exactly one batch, so every load overwrites pages
that the previous batch's apply -- still queued behind other work on the
compute stream -- reads.  Its results match the oracle only if the loads are
ordered after it.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import gather_lora_matmul_amd as L  # noqa: E402
import workloads as W  # noqa: E402
from gather_lora_matmul_amd.synthetic import prepare_shapes, to_device  # noqa: E402

from gpu_helpers import Guarded, check_all, ids_tensor, log  # noqa: E402

PER_BATCH = 12


def _pages(wl, adapters):
    """Pool pages the adapters occupy in every slice (the documented layout)."""
    per16 = 16 // W.ELT_BYTES[wl.dtype]
    P = wl.page_elems
    total = 0
    for a in adapters:
        r = int(wl.ranks[a])
        rs = -(-r // per16) * per16
        for d_in, d_out in wl.slices:
            total += r * -(-d_in // P) + -(-d_out // (P // rs))
    return total


def _pool_and_store(wl, n_pages: int, poison=True):
    """A pool of n_pages pages and a store holding all the workload's adapters."""
    pool = L.lora_pool_create(wl.page_elems, W.DTYPE_CODE[wl.dtype], n_pages, wl.n_adapters,
                              wl.max_rank, wl.slices, shuffle_seed=wl.shuffle_seed,
                              flags=L.LORA_POOL_POISON if poison else 0,
                              act_dtype=W.DTYPE_CODE[wl.act_dtype])
    L.lora_page_table_build(pool)
    store = L.lora_store_create(pool)
    for a in range(wl.n_adapters):
        for s in range(len(wl.slices)):
            A, B = wl.weights(a, s)
            q = wl.qscales(a, s)
            L.lora_store_add(store, a, s, int(wl.ranks[a]), float(wl.scales[a]), A, B,
                             *(q if q is not None else (None, None)))
    return pool, store


def _busy(n=6):
    # enqueue a few milliseconds of unrelated work on the current (compute) stream
    a = torch.randn(2048, 2048, device="cuda")
    for _ in range(n):
        a = a @ a
        a = a / a.abs().max()
    return a


@pytest.mark.parametrize("entry", ["bgmv", "planned"])
@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_loads_overlap_compute_and_evict_lru(entry, dtype):
    ranks = [16, 8, 32, 16] * 12
    wl = W.small_workload(dtype, 1024, 1536, ranks, 1024, n_slices=2, seed=90,
                          act_dtype="bf16" if dtype == "e4m3" else None)
    act = wl.act_dtype
    log("[case] residency %s %s: %d adapters, room for %d" % (entry, dtype, len(ranks), PER_BATCH))
    # room for exactly one batch (every batch has the same rank mix): each
    # batch evicts all of the previous one and loads into its pages
    pool, store = _pool_and_store(wl, _pages(wl, range(PER_BATCH)))
    upload = torch.cuda.Stream()  # default priority
    compute = torch.cuda.current_stream()
    rng = np.random.default_rng(4)
    plans = []
    keep = []
    # every batch's buffers first: the loop below enqueues work without a host wait
    batches = []
    for k in range(6):
        # disjoint from the previous batch: loads evict its adapters
        base = (k % 4) * PER_BATCH
        pick = np.arange(base, base + PER_BATCH)
        ids = np.concatenate([pick, rng.choice(pick, size=24), [-1] * 4]).astype(np.int32)
        rng.shuffle(ids)
        b = W.custom_batch(wl, ids, index=k, zero_y0=(k % 2 == 0))
        xs = [to_device(b.x[s], act) for s in range(2)]
        ys = [Guarded(b.y0[s], act) for s in range(2)]
        batches.append((b, ids, ids_tensor(ids), xs, ys))
    torch.cuda.synchronize()
    try:
        for k, (b, ids, ids_d, xs, ys) in enumerate(batches):
            L.lora_store_ensure(store, ids, upload_stream=upload, compute_stream=compute)
            keep.append(_busy())  # the apply below starts late
            io = [(s, xs[s], ys[s].view) for s in range(2)]
            if entry == "bgmv":
                L.lora_bgmv_apply(pool, io, ids_d, W.DTYPE_CODE[act])
            else:
                plan = L.lora_plan_create(pool, len(ids))
                plans.append(plan)
                L.lora_plan_build(plan, ids)
                ws = prepare_shapes(plan, [[0, 1]])
                L.lora_apply(pool, plan, io, W.DTYPE_CODE[act], workspace=ws)
                keep.append(ws)
        torch.cuda.synchronize()
        st = L.lora_store_get_stats(store)
        assert st["uploads"] == 6 * PER_BATCH * 2, st
        assert st["evictions"] == 5 * PER_BATCH * 2, st
        assert st["resident"] == PER_BATCH and st["registered"] == len(ranks)
        for k, (b, _, _, _, ys) in enumerate(batches):
            check_all(wl, b, {s: ys[s].host() for s in range(2)}, {}, [0, 1], act,
                      "residency %s %s batch %d" % (entry, dtype, k))
    finally:
        torch.cuda.synchronize()
        for p in plans:
            L.lora_plan_destroy(p)
        L.lora_store_destroy(store)
        L.lora_pool_destroy(pool)


def test_lru_keeps_recent_adapters_and_refuses_what_cannot_fit():
    ranks = [16] * 20
    wl = W.small_workload("bf16", 1024, 1024, ranks, 1024, n_slices=2, seed=91)
    log("[case] LRU order, NOMEM, NOT_RESIDENT")
    pool, store = _pool_and_store(wl, _pages(wl, range(8)))
    try:
        up = torch.cuda.Stream()
        L.lora_store_ensure(store, np.arange(0, 8), upload_stream=up)
        L.lora_store_ensure(store, np.array([0, 1, 2, 3]), upload_stream=up)  # 4..7 now least recent
        L.lora_store_ensure(store, np.array([8, 9, 2]), upload_stream=up)      # evicts 4, 5
        torch.cuda.synchronize()
        res = [L.lora_pool_export_entry(pool, a, 0)[0] > 0 for a in range(10)]
        assert res == [True] * 4 + [False, False, True, True, True, True], res
        with pytest.raises(L.LoraError) as e:  # 9 adapters cannot be resident at once
            L.lora_store_ensure(store, np.arange(10, 19), upload_stream=up)
        assert e.value.status == -2
        res2 = [L.lora_pool_export_entry(pool, a, 0)[0] > 0 for a in range(20)]
        assert res2[:10] == res and not any(res2[10:]), "a refused request changed residency"
        with pytest.raises(L.LoraError) as e:  # adapter ids past the store
            L.lora_store_ensure(store, np.array([20]), upload_stream=up)
        assert e.value.status == -1
        # the resident set still computes correctly
        ids = np.array([0, 9, 2, -1, 8, 7], np.int32)
        b = W.custom_batch(wl, ids, zero_y0=True)
        xs = [to_device(b.x[s], "bf16") for s in range(2)]
        ys = [Guarded(b.y0[s], "bf16") for s in range(2)]
        L.lora_bgmv_apply(pool, [(s, xs[s], ys[s].view) for s in range(2)], ids_tensor(ids),
                          L.LORA_BF16)
        torch.cuda.synchronize()
        check_all(wl, b, {s: ys[s].host() for s in range(2)}, {}, [0, 1], "bf16", "after LRU")
    finally:
        torch.cuda.synchronize()
        L.lora_store_destroy(store)
        L.lora_pool_destroy(pool)

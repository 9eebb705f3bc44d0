"""GPU parity of the decode path whose tokens are grouped by adapter on the
device (lora_bgmv_apply_planned): every output row against the fp64 oracle,
exact-integer batches bit-exact, the device-built plan against the host
planner's grouping, skipped ids, adapters missing from one slice, batch sizes
around the tile size and the 1024-token limit.

Every case prints its name and shape before it touches the GPU.  Inputs come
from `workloads` (seeded); expected values only from `oracle`.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import gather_lora_matmul_amd as L  # noqa: E402
import workloads as W  # noqa: E402
from gather_lora_matmul_amd.synthetic import SyntheticPool, to_device  # noqa: E402

from gpu_helpers import Guarded, check_all, exact_compare, ids_tensor, log, reference  # noqa: E402

_POOLS = {}


def pool_for(key, wl, adapters=None):
    if key not in _POOLS:
        log("[setup] pool %s (%s)" % (key, wl.name))
        _POOLS[key] = SyntheticPool(wl, adapters=adapters)
    return _POOLS[key]


@pytest.fixture(scope="module", autouse=True)
def _cleanup():
    yield
    for p in _POOLS.values():
        p.close()
    _POOLS.clear()
    torch.cuda.synchronize()


def workspace(sp, slices, n):
    nb = L.lora_bgmv_planned_workspace_size(sp.handle, slices, n)
    return torch.empty(nb, dtype=torch.uint8, device="cuda")


def run_planned(sp, b, slices, y_dtype, ws=None):
    wl = sp.wl
    n = len(b.ids)
    ids = ids_tensor(b.ids)
    xs = {s: to_device(b.x[s], wl.act_dtype) for s in slices}
    ys = {s: Guarded(b.y0[s], y_dtype) for s in slices}
    if ws is None:
        ws = workspace(sp, slices, n)
    L.lora_bgmv_apply_planned(sp.handle, [(s, xs[s], ys[s].view) for s in slices], ids,
                              W.DTYPE_CODE[y_dtype], ws)
    torch.cuda.synchronize()
    return {s: ys[s].host() for s in slices}, ws


def test_devplan_hetero_decode_full():
    wl = W.make_workload(2)
    log("[case] device-planned hetero decode, 256 tokens x 2 slices")
    sp = pool_for("cfg2", wl)
    b = W.make_batch(wl, 0)
    ys, _ = run_planned(sp, b, [0, 1], wl.dtype)
    check_all(wl, b, ys, {}, [0, 1], wl.dtype, "devplan cfg2")
    # fp32 y accumulated onto a random y0 (the delta gated on its own too)
    b32 = W.make_batch(wl, 1, y_dtype="f32", zero_y0=False)
    ys, _ = run_planned(sp, b32, [1, 0], "f32")
    check_all(wl, b32, ys, {}, [0, 1], "f32", "devplan cfg2 f32")


def test_devplan_plan_matches_host_planner():
    """The plan the device wrote into the workspace groups the tokens and cuts
    the tiles exactly as lora_plan_build does on the host."""
    wl = W.make_workload(2)
    log("[case] device plan vs host plan, hetero decode batch 3")
    sp = pool_for("cfg2", wl)
    b = W.make_batch(wl, 3)
    ys, ws = run_planned(sp, b, [0, 1], wl.dtype)
    raw = ws.cpu().numpy()
    counts = raw[:32].view(np.int32)
    T, nv = int(counts[0]), int(counts[1])
    n = len(b.ids)
    off_perm = 256
    off_items = off_perm + ((4 * n + 255) // 256) * 256
    perm_dev = raw[off_perm:off_perm + 4 * n].view(np.int32)[:nv]
    items_dev = raw[off_items:off_items + 16 * T].view(np.int32).reshape(T, 4)
    plan = L.lora_plan_create(sp.handle, n)
    L.lora_plan_build(plan, b.ids)
    perm_h, items_h = L.lora_plan_export(plan)
    L.lora_plan_destroy(plan)
    valid = int(np.sum(b.ids >= 0))
    assert nv == valid
    assert np.array_equal(perm_dev, perm_h[:valid])
    assert np.array_equal(items_dev, items_h[items_h[:, 3] == 1])
    assert int(counts[2]) == len(set(b.ids[b.ids >= 0].tolist()))
    check_all(wl, b, ys, {}, [0, 1], wl.dtype, "devplan cfg2 batch 3")


@pytest.mark.parametrize("cfg", [1, 2])
def test_devplan_exact_integer_bit_exact(cfg):
    wl = W.make_workload(cfg, exact=True)
    b = W.make_batch(wl, 0, zero_y0=False)
    used = sorted(set(b.ids.tolist()))
    log("[case] device-planned exact cfg=%d adapters=%d" % (cfg, len(used)))
    sp = pool_for(("exact", cfg), wl, adapters=used + list(range(0, wl.n_adapters, 97)))
    slices = list(range(len(wl.slices)))
    ys, _ = run_planned(sp, b, slices, wl.dtype)
    for s in slices:
        exact_compare(ys[s], reference(wl, b, s, wl.dtype), wl.dtype, "devplan exact cfg%d s%d" % (cfg, s))


def _small():
    return W.small_workload("bf16", 1024, 1000, [8, 40, 16, 64, 24], 1024, n_slices=3, seed=21)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 130, 1000, 1024])
def test_devplan_batch_sizes(n):
    """Batches around the 64-token tile and at the 1024-token limit: one
    adapter taking half the tokens (split over several tiles), the others
    mixed, a few skipped; every row of all three slices against the oracle,
    and a second call on the same inputs gives the same bits."""
    wl = _small()
    sp = pool_for("small", wl)
    rng = np.random.default_rng(n)
    ids = rng.integers(0, 5, n).astype(np.int32)
    ids[rng.random(n) < 0.5] = 3
    ids[::17] = -1
    log("[case] device-planned batch n=%d" % n)
    b = W.custom_batch(wl, ids, zero_y0=False)
    ys, ws = run_planned(sp, b, [2, 0, 1], "bf16")
    check_all(wl, b, ys, {}, [0, 1, 2], "bf16", "devplan n=%d" % n)
    ys2, _ = run_planned(sp, b, [2, 0, 1], "bf16", ws=ws)
    for s in range(3):
        assert ys[s].tobytes() == ys2[s].tobytes(), "slice %d not deterministic" % s


def test_devplan_skipped_ids_and_partial_residency():
    """Ids < 0 and at or past max_adapters leave y untouched; an adapter evicted
    from one slice leaves that slice's rows untouched and still applies in the
    others; a batch without any adapter leaves every row untouched."""
    wl = W.small_workload("bf16", 1024, 1000, [8, 40, 16, 64, 24], 1024, n_slices=3, seed=22)
    sp = SyntheticPool(wl)
    try:
        L.lora_pool_evict(sp.handle, 2, 1)
        L.lora_page_table_build(sp.handle)
        ids = np.array([0, -1, 2, 5, 2, 1, 2 ** 31 - 1, 4, 2, -7, 3, 2, 0, 1000, 2], np.int32)
        log("[case] device-planned skipped ids, adapter 2 missing from slice 1")
        b = W.custom_batch(wl, ids, zero_y0=False)
        ys, _ = run_planned(sp, b, [0, 1, 2], "bf16")
        skip = (ids < 0) | (ids >= wl.n_adapters)
        ref_ids = np.where(skip, -1, ids).astype(np.int32)
        for s in range(3):
            assert ys[s][skip].tobytes() == b.y0[s][skip].tobytes()
            rid = np.where(ref_ids == 2, -1, ref_ids) if s == 1 else ref_ids
            rb = W.Batch(ids=rid.astype(np.int32), x=b.x, y0=b.y0)
            check_all(wl, rb, {s: ys[s]}, {}, [s], "bf16", "devplan partial s%d" % s)
        log("[case] device-planned batch without adapters")
        none = np.array([-1, 5, -3, 99], np.int32)
        b0 = W.custom_batch(wl, none, zero_y0=False)
        ys0, _ = run_planned(sp, b0, [0, 1, 2], "bf16")
        for s in range(3):
            assert ys0[s].tobytes() == b0.y0[s].tobytes()
    finally:
        sp.close()


def test_devplan_workspace_checks():
    wl = _small()
    sp = pool_for("small", wl)
    log("[case] device-planned workspace checks")
    n = 8
    b = W.custom_batch(wl, np.arange(n, dtype=np.int32) % 5, zero_y0=True)
    ids = ids_tensor(b.ids)
    x = to_device(b.x[0], "bf16")
    y = to_device(b.y0[0], "bf16")
    nb = L.lora_bgmv_planned_workspace_size(sp.handle, [0], n)
    short = torch.empty(nb - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.LoraError) as ei:
        L.lora_bgmv_apply_planned(sp.handle, [(0, x, y)], ids, L.LORA_BF16, short)
    assert ei.value.status == -1  # LORA_E_ARG
    with pytest.raises(L.LoraError):
        L.lora_bgmv_planned_workspace_size(sp.handle, [0], 1025)
    torch.cuda.synchronize()
    assert np.all(y.cpu().view(torch.int16).numpy() == 0)  # nothing launched


def test_dplan_built_once_applied_to_other_layers():
    """One device plan built from a batch's ids on slices 0 and 1, applied to
    slices 0, 1 and to slices 2, 3 (another layer of the same shapes): every
    row of all four slices against the oracle, the bits equal to the one-shot
    lora_bgmv_apply_planned; a residency change makes the plan stale."""
    wl = W.small_workload("bf16", 1024, 1000, [8, 40, 16, 64, 24], 1024, n_slices=4, seed=23)
    sp = SyntheticPool(wl)
    d = L.lora_dplan_create(sp.handle, 300, [0, 1])
    try:
        rng = np.random.default_rng(9)
        ids = rng.integers(-1, 5, 300).astype(np.int32)
        ids[:120] = 2
        log("[case] device plan built once, applied to two layers, 300 tokens")
        b = W.custom_batch(wl, ids, zero_y0=False)
        idt = ids_tensor(ids)
        xs = {s: to_device(b.x[s], "bf16") for s in range(4)}
        ys = {s: Guarded(b.y0[s], "bf16") for s in range(4)}
        L.lora_dplan_build(d, [0, 1], idt)
        L.lora_dplan_apply(sp.handle, d, [(0, xs[0], ys[0].view), (1, xs[1], ys[1].view)], 300, L.LORA_BF16)
        L.lora_dplan_apply(sp.handle, d, [(2, xs[2], ys[2].view), (3, xs[3], ys[3].view)], 300, L.LORA_BF16)
        torch.cuda.synchronize()
        got = {s: ys[s].host() for s in range(4)}
        check_all(wl, b, got, {}, [0, 1, 2, 3], "bf16", "dplan layers")
        one, _ = run_planned(sp, b, [2, 3], "bf16")
        for s in (2, 3):
            assert got[s].tobytes() == one[s].tobytes(), "slice %d differs from the one-shot call" % s
        L.lora_pool_evict(sp.handle, 4, 3)
        L.lora_page_table_build(sp.handle)
        with pytest.raises(L.LoraError) as ei:
            L.lora_dplan_apply(sp.handle, d, [(2, xs[2], ys[2].view), (3, xs[3], ys[3].view)], 300,
                               L.LORA_BF16)
        assert ei.value.status == -5  # LORA_E_STATE
    finally:
        L.lora_dplan_destroy(d)
        sp.close()

"""Host-side checks of the C ABI (no GPU): exported symbols, pool layout and
page-table contents on a host-only pool, allocator and planner invariants,
error paths."""
import ctypes
import subprocess

import numpy as np
import pytest

import gather_lora_matmul_amd as L
import oracle
import workloads as W
from gather_lora_matmul_amd.synthetic import SyntheticPool


def _declared_symbols():
    import re
    src = open(L.__file__.replace("gather_lora_matmul_amd/__init__.py", "include/lora_mi355x.h")).read()
    return sorted(set(re.findall(r"^(?:lora_status|const char\*)\s+(lora_\w+)\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    decl = _declared_symbols()
    assert len(decl) >= 20
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [s for s in decl if s not in exported]
    assert not missing, missing
    assert set(decl) == set(L.EXPORTS)
    for s in decl:
        assert getattr(L.lib(), s) is not None


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no fallback path: without the built library the binding refuses to load
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "liblora_mi355x.so"))
    with pytest.raises(ImportError, match="not built"):
        L._load()


def test_library_has_gfx950_code_object():
    # the offload bundle of the library built here names its target
    with open(L.LIB_PATH, "rb") as f:
        assert b"amdgcn-amd-amdhsa--gfx950" in f.read()


def _host_pool(wl, **kw):
    return SyntheticPool(wl, host_only=True, **kw)


@pytest.mark.parametrize("cfg_args", [
    ("f32", 256, 256, [4, 8, 8, 16], 256),          # the tiny configuration's shapes
    ("bf16", 48, 40, [5, 3, 13], 32),              # d_in spans 2 pages, odd ranks, ragged B
    ("f16", 64, 104, [16, 1, 9], 64),
    ("e4m3", 96, 72, [5, 16, 33], 64),             # one-byte codes: r_s = rank rounded to 16
])
def test_host_pool_layout_walks_back_to_dense(cfg_args):
    dtype, d_in, d_out, ranks, P = cfg_args
    wl = W.small_workload(dtype, d_in, d_out, ranks, P, n_slices=2)
    with _host_pool(wl) as sp:
        free, _ = L.lora_pool_info(sp.handle)
        image = L.lora_pool_read_pages(sp.handle, 0, sp.n_pages, P, sp.dt)
        seen = set()
        for s in range(2):
            for a in range(len(ranks)):
                r, sc, ap, bp = L.lora_pool_export_entry(sp.handle, a, s)
                assert r == ranks[a] and np.float32(sc) == wl.scales[a]
                per16 = 16 // W.ELT_BYTES[dtype]
                if dtype == "e4m3":  # the per-rank scales come back as uploaded
                    sa, sb = L.lora_pool_export_scales(sp.handle, a, s, r)
                    qa, qb = wl.qscales(a, s)
                    assert sa.tobytes() == qa.tobytes() and sb.tobytes() == qb.tobytes()
                rs = -(-r // per16) * per16
                assert ap.size == r * -(-d_in // P) and bp.size == -(-d_out // (P // rs))
                for pg in np.concatenate([ap, bp]).tolist():
                    assert 0 <= pg < sp.n_pages and pg not in seen
                    seen.add(pg)
                A, B = oracle.walk_adapter(image, dtype, P, d_in, d_out, r, ap, bp)
                A0, B0 = wl.weights(a, s)
                assert A.tobytes() == A0.tobytes() and B.tobytes() == B0.tobytes()
        assert free == sp.n_pages - len(seen)
        # unused pages and page tails are NaN-poisoned
        used = np.zeros(sp.n_pages, bool)
        used[list(seen)] = True
        pages = image.reshape(sp.n_pages, P)
        nan_bits = W.NAN_BITS[dtype]
        if dtype == "f32":
            assert np.all(np.isnan(pages[~used]))
        else:
            assert np.all(pages[~used] == nan_bits)


def test_pages_are_scattered_by_the_seed():
    wl = W.small_workload("bf16", 64, 64, [8] * 6, 64)
    with _host_pool(wl) as sp:
        _, ap, _ = L.lora_pool_export_entry(sp.handle, 0, 0)[1:]
        ap = L.lora_pool_export_entry(sp.handle, 0, 0)[2]
    assert not np.all(np.diff(ap) == 1)


def test_kv_dummy_pages_interleave():
    wl = W.small_workload("bf16", 64, 64, [8] * 6, 64, kv_dummy_ratio=1.0)
    with _host_pool(wl) as sp:
        kv = np.concatenate(sp.kv_pages)
        allp = []
        for a in range(6):
            _, _, ap, bp = L.lora_pool_export_entry(sp.handle, a, 0)
            allp += ap.tolist() + bp.tolist()
        assert len(set(kv.tolist()) & set(allp)) == 0
        assert abs(len(kv) - len(allp)) <= 1


def test_allocator_errors_leave_state_unchanged():
    wl = W.small_workload("f16", 64, 64, [8, 8], 64)
    sp = _host_pool(wl, n_pages=40)
    h = sp.handle
    free0, _ = L.lora_pool_info(h)
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_alloc_pages(h, free0 + 1)
    assert e.value.status == -2
    assert L.lora_pool_info(h)[0] == free0
    ids = L.lora_pool_alloc_pages(h, 3)
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_free_pages(h, np.array([ids[0], ids[0]], np.int32))
    assert e.value.status == -5
    _, _, ap, _ = L.lora_pool_export_entry(h, 0, 0)
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_free_pages(h, ap[:1])
    assert e.value.status == -5
    L.lora_pool_free_pages(h, ids)
    assert L.lora_pool_info(h)[0] == free0
    # double upload, rank out of range, eviction twice
    A, B = wl.weights(0, 0)
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_upload(h, 0, 0, 8, 1.0, A, B)
    assert e.value.status == -5
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_upload(h, 1, 0, 9, 1.0, np.zeros((9, 64), np.uint16), np.zeros((64, 9), np.uint16))
    assert e.value.status == -4
    L.lora_pool_evict(h, 1, 0)
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_evict(h, 1, 0)
    assert e.value.status == -5
    # not enough pages: NOMEM and nothing taken
    big = np.zeros((8, 64), np.uint16)
    free1 = L.lora_pool_info(h)[0]
    L.lora_pool_alloc_pages(h, free1 - 3)
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_upload(h, 1, 0, 8, 1.0, big, np.zeros((64, 8), np.uint16))
    assert e.value.status == -2
    assert L.lora_pool_info(h)[0] == 3
    sp.close()


def test_compute_refuses_host_only_and_stale_tables():
    wl = W.small_workload("bf16", 64, 64, [8], 64)
    with _host_pool(wl) as sp:
        with pytest.raises(L.LoraError) as e:
            L.lib().lora_bgmv_shrink  # exists
            st = L.lib().lora_bgmv_shrink(sp.handle, 0, 16, 16, 1, 16, 8, None)
            L._check(st, "bgmv_shrink")
        assert e.value.status == -5


def test_bad_pool_descriptions():
    for kw, code in [(dict(page_elems=3), -1), (dict(max_rank=200), -4), (dict(max_rank=0), -4),
                     (dict(n_pages=0), -1)]:
        args = dict(page_elems=64, dtype=L.LORA_BF16, n_pages=16, max_adapters=2, max_rank=8,
                    slice_dims=[(64, 64)], flags=L.LORA_POOL_HOST_ONLY)
        args.update(kw)
        with pytest.raises(L.LoraError) as e:
            L.lora_pool_create(**args)
        assert e.value.status == code, kw
    with pytest.raises(L.LoraError):
        L.lora_pool_create(64, L.LORA_BF16, 16, 2, 8, [(60, 64)], flags=L.LORA_POOL_HOST_ONLY)


def _plan_for(wl, ids, l_long=0):
    sp = _host_pool(wl)
    plan = L.lora_plan_create(sp.handle, max(1, len(ids)))
    L.lora_plan_build(plan, np.asarray(ids, np.int32), l_long=l_long, stream=0)
    return sp, plan


def test_planner_groups_the_index_vector_example():
    # tokens 1..4 -> adapters #12, #05, #88, #12 (serving article, SGMV diagram)
    wl = W.small_workload("bf16", 64, 64, [4] * 89, 64)
    sp, plan = _plan_for(wl, [12, 5, 88, 12, -1])
    perm, items = L.lora_plan_export(plan)
    st = L.lora_plan_get_stats(plan)
    assert st["n_groups"] == 4 and st["n_tokens"] == 5
    groups = {}
    for a, start, count, kind in items.tolist():
        groups.setdefault(a, []).extend(perm[start:start + count].tolist())
    assert groups == {12: [0, 3], 5: [1], 88: [2], -1: [4]}
    L.lora_plan_destroy(plan)
    sp.close()


@pytest.mark.parametrize("l_long", [0, 1, 1 << 30])
def test_planner_invariants(l_long):
    rng = np.random.default_rng(7)
    # P = 1024: ranks up to 64 leave >= 16 B rows per page (MFMA tiles);
    # rank 96 does not, and its groups stay short items whatever their length
    ranks = list(rng.choice([8, 16, 64, 40, 96], 50))
    ranks[3], ranks[9] = 64, 96
    wl = W.small_workload("bf16", 64, 64, ranks, 1024)
    ids = np.concatenate([np.full(150, 3), rng.integers(-1, 50, 400), np.full(70, 9)]).astype(np.int32)
    rng.shuffle(ids)
    sp, plan = _plan_for(wl, ids, l_long)
    perm, items = L.lora_plan_export(plan)
    assert sorted(perm.tolist()) == list(range(len(ids)))
    covered = np.zeros(len(ids), int)
    eff = 1 if l_long <= 0 else l_long
    counts = {a: int(np.sum(ids == a)) for a in set(ids.tolist())}

    def tile_layout_ok(a):  # stored B row = rank rounded up to 8 elements
        return 1024 // ((int(ranks[a]) + 7) // 8 * 8) >= 16

    n_tiles = 0
    for a, start, count, kind in items.tolist():
        toks = perm[start:start + count]
        covered[toks] += 1
        assert np.all(ids[toks] == a) or (a == -1 and np.all(ids[toks] < 0))
        assert np.all(np.diff(toks) > 0)           # stable: original order inside a group
        if kind == 1:
            assert a >= 0 and count <= 64 and counts[a] >= eff and tile_layout_ok(a)
            n_tiles += 1
        else:
            assert count <= 4 and (a < 0 or counts[a] < eff or not tile_layout_ok(a))
    if l_long < (1 << 30):
        assert n_tiles > 0 and not any(it[0] == 9 and it[3] == 1 for it in items.tolist())
    assert np.all(covered == 1)
    kinds = items[:, 3]
    assert np.all(np.diff(kinds) <= 0)              # MFMA tiles first
    L.lora_plan_destroy(plan)
    sp.close()


def test_planner_rejects_bad_ids():
    wl = W.small_workload("bf16", 64, 64, [8, 8], 64)
    sp = _host_pool(wl, adapters=[0])
    plan = L.lora_plan_create(sp.handle, 8)
    with pytest.raises(L.LoraError) as e:
        L.lora_plan_build(plan, np.array([0, 1], np.int32), stream=0)
    assert e.value.status == -3
    with pytest.raises(L.LoraError) as e:
        L.lora_plan_build(plan, np.array([0, 2], np.int32), stream=0)
    assert e.value.status == -1
    with pytest.raises(L.LoraError) as e:
        L.lora_plan_build(plan, np.zeros(9, np.int32), stream=0)
    assert e.value.status == -1
    L.lora_plan_destroy(plan)
    sp.close()


def test_workspace_is_sized_per_prepared_shape_and_checked():
    # A planned call needs its launch shape prepared after the plan build, and
    # a caller-owned workspace of at least lora_workspace_size bytes: a short
    # one is LORA_E_ARG before anything else happens.
    wl = W.small_workload("bf16", 256, 520, [16, 64, 5], 256, n_slices=2)
    ids = np.array([0] * 70 + [1] * 17 + [2] * 30 + [-1] * 3, np.int32)
    sp, plan = _plan_for(wl, ids)
    try:
        assert L.lora_plan_get_stats(plan)["n_mfma_items"] > 0
        with pytest.raises(L.LoraError) as e:
            L.lora_workspace_size(plan, [0, 1])
        assert e.value.status == -5  # not prepared
        L.lora_plan_prepare(plan, [0, 1], stream=0)
        L.lora_plan_prepare(plan, [1], stream=0)
        need2 = L.lora_workspace_size(plan, [0, 1])
        need1 = L.lora_workspace_size(plan, [1])
        assert need2 > need1 > 0 and need2 % 16 == 0
        # a shape is the sequence of the slices' dims: [1, 0] has those of [0, 1]
        assert L.lora_workspace_size(plan, [1, 0]) == need2
        fake = 1 << 20  # never dereferenced: every call below fails on the host
        io = (L.Io * 2)(L.Io(0, 0, fake, fake), L.Io(1, 0, fake, fake))
        lib = L.lib()
        st = lib.lora_apply(sp.handle, plan, 2, io, L.LORA_BF16, fake, need2 - 16, None)
        assert st == -1 and "workspace" in L.lora_last_error()
        st = lib.lora_apply(sp.handle, plan, 2, io, L.LORA_BF16, None, need2, None)
        assert st == -1
        st = lib.lora_apply(sp.handle, plan, 2, io, L.LORA_BF16, fake + 8, need2, None)
        assert st == -1 and "aligned" in L.lora_last_error()
        st = lib.lora_sgmv_shrink(sp.handle, plan, 1, fake, fake, 64, fake, need1 - 16, None)
        assert st == -1
        # enough workspace: the host-only pool is refused only now
        st = lib.lora_apply(sp.handle, plan, 2, io, L.LORA_BF16, fake, need2, None)
        assert st == -5 and "host-only" in L.lora_last_error()
        # a new build drops the prepared shapes
        L.lora_plan_build(plan, ids[:50], stream=0)
        with pytest.raises(L.LoraError) as e:
            L.lora_workspace_size(plan, [0, 1])
        assert e.value.status == -5
        st = lib.lora_apply(sp.handle, plan, 2, io, L.LORA_BF16, fake, need2, None)
        assert st == -5 and "prepare" in L.lora_last_error()
    finally:
        L.lora_plan_destroy(plan)
        sp.close()


def test_binding_checks_buffers_before_the_call():
    # The C ABI takes raw pointers; the binding checks element types and sizes
    # first (host tensors suffice: nothing reaches the library).
    torch = pytest.importorskip("torch")
    wl = W.small_workload("bf16", 64, 128, [8, 8], 64, n_slices=2)
    with _host_pool(wl) as sp:
        n = 5
        x = torch.zeros((n, 64), dtype=torch.bfloat16)
        y = torch.zeros((n, 128), dtype=torch.bfloat16)
        ids64 = torch.zeros(n, dtype=torch.int64)
        ids = torch.zeros(n, dtype=torch.int32)
        with pytest.raises(TypeError, match="int32"):
            L.lora_bgmv_apply(sp.handle, [(0, x, y)], ids64, L.LORA_BF16)
        with pytest.raises(TypeError, match="dtype"):
            L.lora_bgmv_apply(sp.handle, [(0, x.float(), y)], ids, L.LORA_BF16)
        with pytest.raises(TypeError, match="dtype"):
            L.lora_bgmv_apply(sp.handle, [(0, x, y)], ids, L.LORA_F32)
        with pytest.raises(ValueError, match="elements"):
            L.lora_bgmv_apply(sp.handle, [(1, x, y[:4])], ids, L.LORA_BF16)
        with pytest.raises(ValueError, match="elements"):
            L.lora_bgmv_shrink(sp.handle, 0, x[:3], ids, torch.zeros((n, 8)))
        with pytest.raises(ValueError, match="elements"):
            L.lora_bgmv_expand(sp.handle, 0, torch.zeros((n, 4)), ids, y, L.LORA_BF16, v_ld=8)
        with pytest.raises(TypeError, match="dtype"):
            L.lora_bgmv_expand(sp.handle, 0, torch.zeros((n, 8), dtype=torch.float64), ids, y,
                               L.LORA_BF16)


def test_fp8_pool_arguments():
    # FP8 pages need 16-bit activations, d_in a multiple of 16 and scaled uploads
    base = dict(page_elems=64, dtype=L.LORA_FP8_E4M3, n_pages=64, max_adapters=2, max_rank=16,
                slice_dims=[(64, 40)], flags=L.LORA_POOL_HOST_ONLY)
    for kw in (dict(act_dtype=L.LORA_FP8_E4M3), dict(act_dtype=L.LORA_F32),
               dict(act_dtype=L.LORA_F16, slice_dims=[(72, 40)])):
        args = dict(base)
        args.update(kw)
        with pytest.raises(L.LoraError) as e:
            L.lora_pool_create(**args)
        assert e.value.status == -1, kw
    with pytest.raises(L.LoraError) as e:  # 16-bit pools keep x in the page dtype
        L.lora_pool_create(64, L.LORA_BF16, 16, 2, 8, [(64, 64)], flags=L.LORA_POOL_HOST_ONLY,
                           act_dtype=L.LORA_F16)
    assert e.value.status == -1
    h = L.lora_pool_create(**dict(base, act_dtype=L.LORA_BF16))
    try:
        A = np.zeros((4, 64), np.uint8)
        B = np.zeros((40, 4), np.uint8)
        with pytest.raises(L.LoraError) as e:
            L.lora_pool_upload(h, 0, 0, 4, 1.0, A, B)
        assert e.value.status == -1 and "scaled" in str(e.value)
        L.lora_pool_upload_scaled(h, 0, 0, 4, 1.0, A, np.ones(4), B, np.full(4, 0.5))
        sa, sb = L.lora_pool_export_scales(h, 0, 0, 4)
        assert np.all(sa == 1.0) and np.all(sb == 0.5)
        with pytest.raises(L.LoraError) as e:
            L.lora_pool_export_scales(h, 1, 0, 4)
        assert e.value.status == -3
    finally:
        L.lora_pool_destroy(h)
    h = L.lora_pool_create(64, L.LORA_BF16, 16, 2, 8, [(64, 64)], flags=L.LORA_POOL_HOST_ONLY)
    try:
        with pytest.raises(L.LoraError) as e:
            L.lora_pool_upload_scaled(h, 0, 0, 4, 1.0, np.zeros((4, 64), np.uint16), np.ones(4),
                                      np.zeros((64, 4), np.uint16), np.ones(4))
        assert e.value.status == -1
    finally:
        L.lora_pool_destroy(h)


def test_x_group_needs_one_x_and_one_d_in():
    # entries of one x_group must name the same x buffer and d_in; the check
    # comes before the pool's state (a host-only pool runs nothing)
    wl = W.small_workload("bf16", 64, 64, [8], 64, n_slices=3)
    wl.slices[2] = (128, 64)
    with _host_pool(wl) as sp:
        lib, a, b = L.lib(), 1 << 20, 2 << 20
        io = (L.Io * 2)(L.Io(0, 1, a, a), L.Io(1, 1, b, b))
        assert lib.lora_bgmv_apply(sp.handle, 2, io, a, 4, L.LORA_BF16, None) == -1
        assert "x_group" in L.lora_last_error()
        io = (L.Io * 2)(L.Io(0, 2, a, a), L.Io(2, 2, a, b))
        assert lib.lora_bgmv_apply(sp.handle, 2, io, a, 4, L.LORA_BF16, None) == -1
        io = (L.Io * 2)(L.Io(0, 1, a, a), L.Io(1, -3, a, b))
        assert lib.lora_bgmv_apply(sp.handle, 2, io, a, 4, L.LORA_BF16, None) == -1
        io = (L.Io * 3)(L.Io(0, 1, a, a), L.Io(2, 0, b, b), L.Io(1, 1, a, b))
        assert lib.lora_bgmv_apply(sp.handle, 3, io, a, 4, L.LORA_BF16, None) == -5  # valid: pool state


def test_device_planned_decode_arguments():
    # lora_bgmv_apply_planned: the workspace bound grows with tokens and
    # slices; pools the MFMA tiles cannot take, more than 1024 tokens and a
    # short or misaligned workspace are refused before anything runs
    wl = W.small_workload("bf16", 1024, 1000, [8, 40, 16, 64, 24], 1024, n_slices=3, seed=21)
    sp = _host_pool(wl)
    try:
        n1 = L.lora_bgmv_planned_workspace_size(sp.handle, [0], 64)
        n2 = L.lora_bgmv_planned_workspace_size(sp.handle, [0, 2], 64)
        n3 = L.lora_bgmv_planned_workspace_size(sp.handle, [0, 2], 256)
        assert 0 < n1 < n2 < n3 and n3 % 256 == 0
        with pytest.raises(L.LoraError) as e:
            L.lora_bgmv_planned_workspace_size(sp.handle, [0], 1025)
        assert e.value.status == -1
        with pytest.raises(L.LoraError) as e:
            L.lora_bgmv_planned_workspace_size(sp.handle, [3], 8)
        assert e.value.status == -1
        fake = 1 << 20  # never dereferenced: every call below fails on the host
        io = (L.Io * 2)(L.Io(0, 0, fake, fake), L.Io(2, 0, fake, fake))
        lib = L.lib()
        st = lib.lora_bgmv_apply_planned(sp.handle, 2, io, fake, 64, L.LORA_BF16, fake, n2 - 256, None)
        assert st == -1 and "workspace" in L.lora_last_error()
        st = lib.lora_bgmv_apply_planned(sp.handle, 2, io, fake, 64, L.LORA_BF16, fake + 16, n2, None)
        assert st == -1 and "aligned" in L.lora_last_error()
        st = lib.lora_bgmv_apply_planned(sp.handle, 2, io, fake, 64, L.LORA_BF16, fake, n2, None)
        assert st == -5 and "host-only" in L.lora_last_error()
        assert lib.lora_bgmv_apply_planned(sp.handle, 2, io, fake, 0, L.LORA_BF16, None, 0, None) == 0
    finally:
        sp.close()
    # pages the MFMA tiles cannot take: fp32, FP8, fewer than 16 B rows per page
    for args in [("f32", 256, 256, [4, 8], 256), ("e4m3", 256, 256, [8, 16], 256),
                 ("bf16", 512, 512, [8, 64], 512)]:
        sp = _host_pool(W.small_workload(*args))
        try:
            with pytest.raises(L.LoraError) as e:
                L.lora_bgmv_planned_workspace_size(sp.handle, [0], 8)
            assert e.value.status == -7, args
        finally:
            sp.close()


def test_device_plan_handle_arguments():
    # lora_dplan_*: created for slice shapes, built on slices of those shapes,
    # applied only to launches of those shapes, never before a build, refused
    # on host-only pools before anything runs
    wl = W.make_workload(2)  # slices 4096x4096 and 4096x11008
    sp = _host_pool(wl, adapters=[0, 1, 2])
    try:
        d = L.lora_dplan_create(sp.handle, 256, [0, 1])
        lib = L.lib()
        fake = 1 << 20  # never dereferenced
        io01 = (L.Io * 2)(L.Io(0, 0, fake, fake), L.Io(1, 0, fake, fake))
        io10 = (L.Io * 2)(L.Io(1, 0, fake, fake), L.Io(0, 0, fake, fake))
        assert lib.lora_dplan_apply(sp.handle, d, 2, io01, L.LORA_BF16, None) == -5  # not built
        assert "not built" in L.lora_last_error()
        assert lib.lora_dplan_build(d, 2, io10, fake, 64, None) == -1  # shapes swapped
        assert lib.lora_dplan_build(d, 2, io01, fake, 257, None) == -1  # past max_tokens
        assert lib.lora_dplan_build(d, 1, io01, fake, 64, None) == -1   # slice count
        st = lib.lora_dplan_build(d, 2, io01, fake, 64, None)
        assert st == -5 and "host-only" in L.lora_last_error()
        assert lib.lora_dplan_build(d, 2, io01, None, 0, None) == -5
        L.lora_dplan_destroy(d)
        with pytest.raises(L.LoraError) as e:
            L.lora_dplan_create(sp.handle, 1025, [0])
        assert e.value.status == -1
    finally:
        sp.close()
    sp = _host_pool(W.small_workload("f32", 256, 256, [4, 8], 256))
    try:
        with pytest.raises(L.LoraError) as e:
            L.lora_dplan_create(sp.handle, 8, [0])
        assert e.value.status == -7
    finally:
        sp.close()

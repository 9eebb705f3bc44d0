"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name, config and seed before it touches the GPU.  Inputs
come from `workloads` (seeded); expected values only from `oracle`.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import gather_lora_matmul_amd as L  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gather_lora_matmul_amd.synthetic import (SyntheticPool, from_device, prepare_shapes,  # noqa: E402
                                              to_device)

from gpu_helpers import (Guarded, check_all, compare, exact_compare, ids_tensor, log,  # noqa: E402
                         reference, run_bgmv, run_sgmv)

_POOLS = {}


def pool_for(key, wl, adapters=None, **kw):
    if key not in _POOLS:
        log("[setup] pool %s (%s, %d adapters)" % (key, wl.name, wl.n_adapters if adapters is None
                                                   else len(set(adapters))))
        _POOLS[key] = SyntheticPool(wl, adapters=adapters, **kw)
    return _POOLS[key]


@pytest.fixture(scope="module", autouse=True)
def _cleanup():
    yield
    for p in _POOLS.values():
        p.close()
    _POOLS.clear()
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# page-table resolution and gather: bit exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [("f32", 256, 256, [4, 8, 8, 16], 256), ("bf16", 48, 40, [5, 3, 13], 32),
                                   ("f16", 4096, 11008, [16, 64, 8], 4096)])
def test_gather_and_resolve_bit_exact(shape):
    dtype, d_in, d_out, ranks, P = shape
    log("[case] gather/resolve %s" % (shape,))
    wl = W.small_workload(dtype, d_in, d_out, ranks, P, n_slices=2, kv_dummy_ratio=1.0)
    sp = SyntheticPool(wl)
    try:
        elt = 4 if dtype == "f32" else 2
        sd = np.float32 if dtype == "f32" else np.uint16
        for s in range(2):
            for a in range(len(ranks)):
                r = ranks[a]
                A = torch.zeros((r, d_in), dtype=torch.int32 if elt == 4 else torch.int16, device="cuda")
                B = torch.zeros((d_out, r), dtype=A.dtype, device="cuda")
                L.lora_debug_gather(sp.handle, s, a, A, B)
                torch.cuda.synchronize()
                A0, B0 = wl.weights(a, s)
                assert A.cpu().numpy().tobytes() == A0.tobytes()
                assert B.cpu().numpy().tobytes() == B0.tobytes()
            ids = np.array([2, -1, 0, 1, 1], np.int32) % len(ranks)
            ids[1] = -1
            npa = -(-d_in // P)
            aoff = torch.zeros((len(ids), sp.max_rank * npa), dtype=torch.int64, device="cuda")
            boff = torch.zeros((len(ids), d_out), dtype=torch.int64, device="cuda")
            L.lora_debug_resolve(sp.handle, s, ids_tensor(ids), aoff, boff)
            torch.cuda.synchronize()
            aoff, boff = aoff.cpu().numpy(), boff.cpu().numpy()
            for i, a in enumerate(ids.tolist()):
                if a < 0:
                    assert np.all(aoff[i] == -1) and np.all(boff[i] == -1)
                    continue
                r, _, ap, bp = L.lora_pool_export_entry(sp.handle, a, s)
                per16 = 16 // elt
                rs = -(-r // per16) * per16
                rpp = P // rs
                want_a = np.full(sp.max_rank * npa, -1, np.int64)
                want_a[: r * npa] = ap.astype(np.int64) * P * elt
                m = np.arange(d_out)
                want_b = (bp[m // rpp].astype(np.int64) * P + (m % rpp) * rs) * elt
                assert np.array_equal(aoff[i], want_a)
                assert np.array_equal(boff[i], want_b)
    finally:
        sp.close()


# ---------------------------------------------------------------------------
# BGMV
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["split", "fused"])
@pytest.mark.parametrize("ydt", ["own", "f32"])
def test_bgmv_tiny(mode, ydt):
    wl = W.make_workload(0)
    y_dtype = wl.dtype if ydt == "own" else "f32"
    log("[case] tiny bgmv mode=%s y=%s seed=%d" % (mode, y_dtype, wl.seed))
    sp = pool_for("tiny", wl)
    for bi in range(3):
        b = W.make_batch(wl, bi, y_dtype=y_dtype, zero_y0=(bi != 2))
        ys, vs = run_bgmv(sp, b, [0], y_dtype, mode, return_v=True)
        check_all(wl, b, ys, vs, [0], y_dtype, "tiny b%d" % bi)


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_bgmv_llama7b_decode_full(mode):
    wl = W.make_workload(1)
    log("[case] llama7b decode bgmv full mode=%s" % mode)
    sp = pool_for("cfg1", wl)
    b = W.make_batch(wl, 0)
    ys, vs = run_bgmv(sp, b, [0, 1, 2, 3], wl.dtype, mode, return_v=True)
    check_all(wl, b, ys, vs, [0, 1, 2, 3], wl.dtype, "cfg1 %s" % mode)


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_bgmv_hetero_decode_full(mode):
    wl = W.make_workload(2)
    log("[case] hetero decode bgmv full mode=%s" % mode)
    sp = pool_for("cfg2", wl)
    b = W.make_batch(wl, 0)
    ys, vs = run_bgmv(sp, b, [0, 1], wl.dtype, mode, return_v=True)
    check_all(wl, b, ys, vs, [0, 1], wl.dtype, "cfg2 %s" % mode)
    # fp32 output accumulated onto a random y0: gated against the unrounded
    # result and, as a delta, against the oracle's delta
    b32 = W.make_batch(wl, 1, y_dtype="f32", zero_y0=False)
    ys, vs = run_bgmv(sp, b32, [1], "f32", mode, return_v=True)
    check_all(wl, b32, ys, vs, [1], "f32", "cfg2 f32 %s" % mode)


@pytest.mark.parametrize("cfg", [0, 1, 2])
@pytest.mark.parametrize("mode", ["split", "fused"])
def test_bgmv_exact_integer_bit_exact(cfg, mode):
    wl = W.make_workload(cfg, exact=True)
    b = W.make_batch(wl, 0, zero_y0=False)
    used = sorted(set(b.ids.tolist()))
    log("[case] exact bgmv cfg=%d mode=%s adapters=%d" % (cfg, mode, len(used)))
    sp = pool_for(("exact", cfg), wl, adapters=used + list(range(0, wl.n_adapters, 97)))
    ys, vs = run_bgmv(sp, b, list(range(len(wl.slices))), wl.dtype, mode, return_v=True)
    for s in range(len(wl.slices)):
        y_ref, v_ref = reference(wl, b, s, wl.dtype, return_v=True)
        exact_compare(ys[s], y_ref, wl.dtype, "exact cfg%d s%d" % (cfg, s))
        if s in vs:  # integer v: exact in fp32 whatever the summation order
            assert np.array_equal(vs[s].astype(np.float64), v_ref), "exact cfg%d s%d v" % (cfg, s)


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_bgmv_negative_and_out_of_table_ids(mode):
    # ids < 0 skip the token (the reference loop's rule); ids at or past
    # max_adapters are treated the same way by the kernels (no read past the
    # adapter table): y bit-identical, v zero
    wl = W.make_workload(2)
    sp = pool_for("cfg2", wl)
    b = W.make_batch(wl, 2, zero_y0=False, n_tokens=32)
    b.ids[::3] = -1
    b.ids[1::7] = wl.n_adapters
    b.ids[2::11] = 2 ** 31 - 1
    b.ids[5] = -(2 ** 31)
    log("[case] negative and out-of-table ids, %s" % mode)
    ys, vs = run_bgmv(sp, b, [0, 1], wl.dtype, mode, return_v=True)
    skip = (b.ids < 0) | (b.ids >= wl.n_adapters)
    assert skip.sum() >= 12
    ref_b = W.Batch(ids=np.where(skip, -1, b.ids).astype(np.int32), x=b.x, y0=b.y0)
    for s in (0, 1):
        assert ys[s][skip].tobytes() == b.y0[s][skip].tobytes()
        if s in vs:
            assert np.all(vs[s][skip] == 0)
    check_all(wl, ref_b, ys, vs, [0, 1], wl.dtype, "skipped ids %s" % mode)


def test_bgmv_zero_token_scale():
    # a token-scale override of 0 leaves y bit-identical (finite data)
    wl = W.make_workload(2)
    sp = pool_for("cfg2", wl)
    b = W.make_batch(wl, 2, zero_y0=False, n_tokens=32)
    b.ids[::3] = -1
    log("[case] zero token scale")
    ids = ids_tensor(b.ids)
    x = to_device(b.x[1], wl.dtype)
    y = Guarded(b.y0[1], wl.dtype)
    v = torch.zeros((32, sp.max_rank), dtype=torch.float32, device="cuda")
    L.lora_bgmv_shrink(sp.handle, 1, x, ids, v)
    L.lora_bgmv_expand(sp.handle, 1, v, ids, y.view, W.DTYPE_CODE[wl.dtype],
                       token_scale=torch.zeros(32, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert y.host().tobytes() == b.y0[1].tobytes()
    assert np.all(v.cpu().numpy()[b.ids < 0] == 0)


@pytest.mark.parametrize("cfg", [1, 5])
@pytest.mark.parametrize("n", [64, 256])
def test_bgmv_shared_x_groups(cfg, n):
    """q, k and v reading one x (x_group 1) and o its own: 256 tokens give one
    block per (group, token) that reads x once, 64 tokens one block per
    (slice, token); every row matches the oracle and the same buffers without
    groups give the same bits."""
    wl = W.make_workload(cfg)
    act = wl.act_dtype
    log("[case] shared-x groups cfg=%d n=%d" % (cfg, n))
    sp = pool_for("cfg%d" % cfg, wl)
    b = W.make_batch(wl, 2, n_tokens=n)
    b.x[1] = b.x[0]
    b.x[2] = b.x[0]
    ids = ids_tensor(b.ids)
    xs = [to_device(b.x[0], act)] * 3 + [to_device(b.x[3], act)]
    out = {}
    for grouped in (True, False):
        ys = [Guarded(b.y0[s], act) for s in range(4)]
        io = [(s, xs[s], ys[s].view, 1 if (grouped and s < 3) else 0) for s in range(4)]
        L.lora_bgmv_apply(sp.handle, io, ids, W.DTYPE_CODE[act])
        torch.cuda.synchronize()
        out[grouped] = {s: ys[s].host() for s in range(4)}
    check_all(wl, b, out[True], {}, [0, 1, 2, 3], act, "shared x cfg%d" % cfg)
    for s in range(4):
        assert out[True][s].tobytes() == out[False][s].tobytes(), "slice %d differs" % s


def test_bgmv_shared_x_multi_page_rows():
    # A rows over two pages take the general body inside a group (x read per
    # slice there); results still match
    wl = W.small_workload("bf16", 512, 264, [8, 40, 16], 256, n_slices=3, seed=12)
    sp = pool_for(("shared_mp",), wl)
    ids = np.array([0, 2, 1, -1, 2, 2, 0, 1] * 3, np.int32)
    b = W.custom_batch(wl, ids, zero_y0=True)
    b.x[1] = b.x[0]
    log("[case] shared-x multi-page rows")
    xs = [to_device(b.x[0], "bf16"), None, to_device(b.x[2], "bf16")]
    xs[1] = xs[0]
    ys = [Guarded(b.y0[s], "bf16") for s in range(3)]
    L.lora_bgmv_apply(sp.handle, [(0, xs[0], ys[0].view, 7), (2, xs[2], ys[2].view, 0),
                                  (1, xs[1], ys[1].view, 7)], ids_tensor(ids), L.LORA_BF16)
    torch.cuda.synchronize()
    check_all(wl, b, {s: ys[s].host() for s in range(3)}, {}, [0, 1, 2], "bf16", "shared x mp")


@pytest.mark.parametrize("n", [129, 500, 513])
def test_bgmv_batch_independent_bits(n):
    """Larger fused batches with repeated, skipped and out-of-table ids and n
    not a multiple of 8 match the oracle, and every token's bits equal those of
    the same token in a smaller batch (a token's result does not depend on
    the batch around it or on the launch shape)."""
    wl = W.make_workload(2)
    sp = pool_for("cfg2", wl)
    b = W.make_batch(wl, 4, zero_y0=False, n_tokens=n)
    b.ids[::13] = -1
    b.ids[5::17] = wl.n_adapters
    b.ids[7] = 2 ** 31 - 1
    b.ids[n // 2: n // 2 + 40] = b.ids[n // 2]  # a long run of one adapter
    log("[case] batch-independent bits n=%d, %d distinct ids" % (n, len(set(b.ids.tolist()))))
    ys = run_bgmv(sp, b, [0, 1], wl.dtype, "fused")
    skip = (b.ids < 0) | (b.ids >= wl.n_adapters)
    ref_b = W.Batch(ids=np.where(skip, -1, b.ids).astype(np.int32), x=b.x, y0=b.y0)
    check_all(wl, ref_b, ys, {}, [0, 1], wl.dtype, "batch bits n=%d" % n)
    step = 100
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        sub = W.Batch(ids=b.ids[lo:hi].copy(), x=[x[lo:hi] for x in b.x],
                      y0=[y[lo:hi] for y in b.y0])
        ysub = run_bgmv(sp, sub, [0, 1], wl.dtype, "fused")
        for s in (0, 1):
            assert ysub[s].tobytes() == ys[s][lo:hi].tobytes(), "tokens %d..%d slice %d" % (lo, hi, s)


def test_bgmv_deterministic_and_placement_independent():
    wl = W.make_workload(2)
    b = W.make_batch(wl, 3, n_tokens=64)
    used = sorted(set(b.ids.tolist()))
    log("[case] determinism / shuffle invariance")
    sp = pool_for("cfg2", wl)
    y1 = run_bgmv(sp, b, [0, 1], wl.dtype, "fused")
    y2 = run_bgmv(sp, b, [0, 1], wl.dtype, "fused")
    wl2 = W.make_workload(2)
    wl2.shuffle_seed = 99991
    sp2 = SyntheticPool(wl2, adapters=used)
    try:
        y3 = run_bgmv(sp2, b, [0, 1], wl.dtype, "fused")
    finally:
        sp2.close()
    for s in range(2):
        assert y1[s].tobytes() == y2[s].tobytes()
        assert y1[s].tobytes() == y3[s].tobytes()


# ---------------------------------------------------------------------------
# SGMV / fused apply
# ---------------------------------------------------------------------------
SMALL_SGMV = [
    # dtype, d_in, d_out, ranks, P, ids
    ("bf16", 256, 520, [16, 64, 5, 128], 256, [0] * 70 + [1] * 17 + [2] * 3 + [3] * 130 + [-1] * 5),
    ("f16", 512, 264, [8, 40, 1], 256, [1] * 33 + [0, 2, 1, 0] * 9 + [2] * 16),
    ("f32", 256, 256, [4, 8, 8, 16], 256, [0, 1, 2, 3] * 10 + [3] * 20),
    # pages large enough for every rank on MFMA tiles; A rows over two pages
    ("bf16", 2304, 1000, [128, 16, 64, 5, 96], 2048,
     [0] * 150 + [1] * 65 + [2] * 7 + [3] * 1 + [4] * 40 + [-1] * 3),
    # groups of at most 16 tokens at every rank band (wide expand steps of 4 and
    # 2 chunks), d_out not a multiple of a step, plus one large group
    ("bf16", 2048, 1000, [128, 96, 64, 33, 8, 16], 2048,
     [0] * 5 + [1] * 16 + [2] * 9 + [3] * 1 + [4] * 12 + [0] * 3 + [5] * 80 + [-1] * 2),
]


@pytest.mark.parametrize("case", range(len(SMALL_SGMV)))
@pytest.mark.parametrize("mode", ["split", "fused"])
@pytest.mark.parametrize("l_long", [0, 16, 1 << 30])
def test_sgmv_small(case, mode, l_long):
    dtype, d_in, d_out, ranks, P, ids = SMALL_SGMV[case]
    log("[case] sgmv small %d mode=%s l_long=%d" % (case, mode, l_long))
    wl = W.small_workload(dtype, d_in, d_out, ranks, P, n_slices=2, seed=40 + case)
    rng = np.random.default_rng(case)
    ids = np.array(ids, np.int32)
    rng.shuffle(ids)
    b = W.custom_batch(wl, ids, zero_y0=True)
    sp = pool_for(("small", case), wl)
    ys, st, vs = run_sgmv(sp, b, [0, 1], dtype, mode, l_long, return_v=True)
    if dtype != "f32" and l_long == 0:
        assert st["n_mfma_items"] > 0
    check_all(wl, b, ys, vs, [0, 1], dtype, "sgmv small %d %s l_long=%d" % (case, mode, l_long))


@pytest.mark.parametrize("case", [0, 3, 4])
@pytest.mark.parametrize("mode", ["split", "fused"])
def test_sgmv_f32_output(case, mode):
    """16-bit pool, fp32 y (accumulated from a random y0): the MFMA tiles'
    fp32-output expand (64-row and wide steps) against the unrounded oracle."""
    dtype, d_in, d_out, ranks, P, ids = SMALL_SGMV[case]
    log("[case] sgmv small %d f32 y mode=%s" % (case, mode))
    wl = W.small_workload(dtype, d_in, d_out, ranks, P, n_slices=2, seed=40 + case)
    ids = np.array(ids, np.int32)
    np.random.default_rng(100 + case).shuffle(ids)
    b = W.custom_batch(wl, ids, y_dtype="f32", zero_y0=False)
    sp = pool_for(("small", case), wl)
    ys, st, vs = run_sgmv(sp, b, [0, 1], "f32", mode, return_v=True)
    assert st["n_mfma_items"] > 0
    check_all(wl, b, ys, vs, [0, 1], "f32", "sgmv small %d f32 %s" % (case, mode))


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_sgmv_exact_small_bit_exact(mode):
    wl = W.small_workload("bf16", 512, 328, [16, 64, 5, 128, 33], 256, n_slices=1, exact=True, seed=77)
    ids = np.array([0] * 90 + [1] * 20 + [2] * 40 + [3] * 70 + [4] * 3 + [-1] * 4, np.int32)
    np.random.default_rng(1).shuffle(ids)
    b = W.custom_batch(wl, ids)
    log("[case] sgmv exact small mode=%s" % mode)
    sp = pool_for("exact_small", wl)
    ys, st, vs = run_sgmv(sp, b, [0], "bf16", mode, return_v=True)
    assert st["n_mfma_items"] > 0
    y_ref, v_ref = reference(wl, b, 0, "bf16", return_v=True)
    exact_compare(ys[0], y_ref, "bf16", "sgmv exact small")
    if vs:
        assert np.array_equal(vs[0].astype(np.float64), v_ref), "sgmv exact small v"
    y_b = run_bgmv(sp, b, [0], "bf16", "fused")[0]
    assert y_b.tobytes() == ys[0].tobytes()


def test_sgmv_plan_reuse_repeated_launches():
    # one plan, several launches in a row (fused, split, fused: the workspace of
    # partial tiles is reused) -- all bit-identical
    dtype, d_in, d_out, ranks, P, ids = SMALL_SGMV[0]
    log("[case] sgmv plan reuse")
    wl = W.small_workload(dtype, d_in, d_out, ranks, P, n_slices=2, seed=40)
    ids = np.array(ids, np.int32)
    np.random.default_rng(3).shuffle(ids)
    b = W.custom_batch(wl, ids)
    sp = pool_for(("small", 0), wl)
    n = len(ids)
    plan = L.lora_plan_create(sp.handle, n)
    try:
        L.lora_plan_build(plan, b.ids)
        ws = prepare_shapes(plan, [[0, 1], [0], [1]])
        xs = [to_device(b.x[s], dtype) for s in range(2)]
        ydt = W.DTYPE_CODE[dtype]
        outs = []
        for rep in range(5):
            ys = [Guarded(b.y0[s], dtype) for s in range(2)]
            if rep in (2, 3):
                v = torch.zeros((n, sp.max_rank), device="cuda")
                for s in range(2):
                    L.lora_sgmv_shrink(sp.handle, plan, s, xs[s], v, workspace=ws)
                    L.lora_sgmv_expand(sp.handle, plan, s, v, ys[s].view, ydt)
            else:
                L.lora_apply(sp.handle, plan, [(s, xs[s], ys[s].view) for s in range(2)], ydt,
                             workspace=ws)
            torch.cuda.synchronize()
            outs.append([ys[s].host() for s in range(2)])
    finally:
        L.lora_plan_destroy(plan)
    for s in range(2):
        compare(outs[0][s], reference(wl, b, s, dtype), dtype, "plan reuse s%d" % s)
        for rep in range(1, 5):
            assert outs[rep][s].tobytes() == outs[0][s].tobytes(), "launch %d differs" % rep


def test_empty_batches_and_tokens_without_adapters():
    """Empty batches: every entry point returns and writes nothing.  A batch in
    which no token has an adapter leaves y bit-identical (BGMV and planned)."""
    log("[case] empty batches, all ids -1")
    wl = W.small_workload("bf16", 512, 264, [8, 40, 16], 256, n_slices=2, seed=9)
    sp = pool_for(("edge",), wl)
    n = 37
    b = W.custom_batch(wl, np.full(n, -1, np.int32))  # random y0
    x = to_device(b.x[0], "bf16")
    y = Guarded(b.y0[0], "bf16")
    v = Guarded(np.full((n, sp.max_rank), np.nan, np.float32), "f32")
    plan = L.lora_plan_create(sp.handle, n)
    try:
        L.lora_bgmv_apply(sp.handle, [(0, x, y.view)], ids_tensor(np.zeros(0, np.int32)), L.LORA_BF16)
        L.lora_plan_build(plan, np.zeros(0, np.int32))
        assert prepare_shapes(plan, [[0]]) is None  # an empty plan needs no workspace
        L.lora_apply(sp.handle, plan, [(0, x, y.view)], L.LORA_BF16)
        L.lora_sgmv_shrink(sp.handle, plan, 0, x, v.view, sp.max_rank)
        L.lora_sgmv_expand(sp.handle, plan, 0, v.view, y.view, L.LORA_BF16, v_ld=sp.max_rank)
        torch.cuda.synchronize()
        assert np.array_equal(y.host(), b.y0[0])
        assert np.all(np.isnan(v.host())), "an empty plan wrote v"
        L.lora_bgmv_apply(sp.handle, [(0, x, y.view)], ids_tensor(b.ids), L.LORA_BF16)
        L.lora_plan_build(plan, b.ids)
        ws = prepare_shapes(plan, [[0]])
        L.lora_apply(sp.handle, plan, [(0, x, y.view)], L.LORA_BF16, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(y.host(), b.y0[0])
    finally:
        L.lora_plan_destroy(plan)


@pytest.mark.parametrize("entry", ["bgmv", "planned"])
def test_fused_apply_max_slices(entry):
    """LORA_MAX_IO (8) slices in one fused call match the oracle; a ninth is
    refused before anything is written."""
    log("[case] fused apply with 8 slices (%s)" % entry)
    wl = W.small_workload("f16", 256, 520, [8, 16, 33], 256, n_slices=9, seed=10)
    sp = pool_for(("max_io",), wl)
    ids = np.array([0, 2, -1, 1, 1, 0, 2, 2, 1, 0, 2] * 3, np.int32)
    b = W.custom_batch(wl, ids, zero_y0=True)
    xs = [to_device(b.x[s], "f16") for s in range(9)]
    ys = [Guarded(b.y0[s], "f16") for s in range(9)]
    plan = L.lora_plan_create(sp.handle, len(ids)) if entry == "planned" else None
    try:
        def call(k):
            io = [(s, xs[s], ys[s].view) for s in range(k)]
            if plan is None:
                L.lora_bgmv_apply(sp.handle, io, ids_tensor(ids), L.LORA_F16)
            else:
                L.lora_apply(sp.handle, plan, io, L.LORA_F16, workspace=ws)
        ws = None
        if plan is not None:
            L.lora_plan_build(plan, ids)
            ws = prepare_shapes(plan, [list(range(8))])
        with pytest.raises(L.LoraError):
            call(9)
        call(8)
        torch.cuda.synchronize()
        for s in range(8):
            compare(ys[s].host(), reference(wl, b, s, "f16"), "f16", "max slices %s s%d" % (entry, s))
        assert np.array_equal(ys[8].host(), b.y0[8])
    finally:
        if plan is not None:
            L.lora_plan_destroy(plan)


def test_plan_layouts_across_launch_shapes():
    """One plan, calls over more distinct launch shapes (slice sets) than the
    plan keeps layouts for: every call matches the oracle, and a shape that
    comes back after its layout was evicted gives bit-identical results."""
    log("[case] plan layouts across launch shapes")
    shapes = [(256, 256), (512, 264), (256, 520), (768, 256), (512, 512), (256, 1000)]
    ranks = np.array([16, 40, 8, 64, 33], np.int32)
    wl = W.Workload("custom", "bgmv", "bf16", 1024, shapes, ranks,
                    np.array([16.0 / r for r in ranks], np.float32), 77, shuffle_seed=11,
                    pool_slack=2.0, kv_dummy_ratio=0.0)
    ids = np.array([0] * 70 + [1] * 9 + [2] * 33 + [3] * 3 + [4] * 20 + [-1] * 2, np.int32)
    np.random.default_rng(5).shuffle(ids)
    b = W.custom_batch(wl, ids, zero_y0=True)
    sp = pool_for(("layouts",), wl)
    n = len(ids)
    plan = L.lora_plan_create(sp.handle, n)
    try:
        L.lora_plan_build(plan, ids)
        xs = [to_device(b.x[s], "bf16") for s in range(len(shapes))]
        refs = {}
        first = {}
        sets = [[0], [1], [0, 2], [3], [4, 5], [1, 2, 3], [0], [5], [0, 2], [2, 4, 5, 1]]
        for k, sl in enumerate(sets):
            ys = [Guarded(b.y0[s], "bf16") for s in sl]
            if k % 3 == 2:  # split calls use the layouts of their single slices
                v_ld = sp.max_rank
                for j, s in enumerate(sl):
                    # preparing more shapes than the plan keeps replaces the
                    # least recently used one
                    ws = prepare_shapes(plan, [[s]])
                    v = Guarded(np.full((n, v_ld), np.nan, np.float32), "f32")
                    L.lora_sgmv_shrink(sp.handle, plan, s, xs[s], v.view, v_ld, workspace=ws)
                    L.lora_sgmv_expand(sp.handle, plan, s, v.view, ys[j].view, L.LORA_BF16, v_ld=v_ld)
                    v.host()
            else:
                ws = prepare_shapes(plan, [sl])
                L.lora_apply(sp.handle, plan, [(s, xs[s], ys[j].view) for j, s in enumerate(sl)],
                             L.LORA_BF16, workspace=ws)
            torch.cuda.synchronize()
            for j, s in enumerate(sl):
                got = ys[j].host()
                if s not in refs:
                    refs[s] = reference(wl, b, s, "bf16")
                compare(got, refs[s], "bf16", "layouts call %d slice %d" % (k, s))
                key = (tuple(sl), s, k % 3 == 2)
                if key in first:
                    assert np.array_equal(first[key], got), "call %d slice %d not bit-identical" % (k, s)
                first.setdefault(key, got)
    finally:
        L.lora_plan_destroy(plan)


def test_sgmv_llama13b_prefill_full():
    # every row of both slices, split (with v) and fused
    wl = W.make_workload(3)
    b = W.make_batch(wl, 0)
    log("[case] llama13b prefill sgmv full, %d tokens" % len(b.ids))
    sp = pool_for("cfg3", wl)
    for mode in ("split", "fused"):
        ys, st, vs = run_sgmv(sp, b, [0, 1], wl.dtype, mode, return_v=True)
        assert st["n_mfma_items"] > 0
        check_all(wl, b, ys, vs, [0, 1], wl.dtype, "cfg3 %s" % mode)


def test_mixed_llama70b_full():
    # every row (4096 prefill + 512 decode tokens) of both slices, split and fused
    wl = W.make_workload(4)
    b = W.make_batch(wl, 0)
    log("[case] llama70b mixed apply full, %d tokens" % len(b.ids))
    sp = pool_for("cfg4", wl)
    for mode in ("split", "fused"):
        ys, st, vs = run_sgmv(sp, b, [0, 1], wl.dtype, mode, return_v=True)
        assert st["n_mfma_items"] > 0
        check_all(wl, b, ys, vs, [0, 1], wl.dtype, "cfg4 %s" % mode)


@pytest.mark.parametrize("cfg", [1, 2])
@pytest.mark.parametrize("mode", ["split", "fused"])
def test_planned_decode_batches_full(cfg, mode):
    # The decode batches with their ids known on the host, run as a plan: every
    # adapter group (one token each, or up to 16 in the heterogeneous batch)
    # becomes an MFMA tile on the wide expand steps; every token checked.
    wl = W.make_workload(cfg)
    b = W.make_batch(wl, 0)
    slices = list(range(len(wl.slices)))
    log("[case] planned decode cfg=%d mode=%s, %d tokens" % (cfg, mode, len(b.ids)))
    sp = pool_for("cfg%d" % cfg, wl)
    ys, st, vs = run_sgmv(sp, b, slices, wl.dtype, mode, return_v=True)
    assert st["n_mfma_items"] > 0
    check_all(wl, b, ys, vs, slices, wl.dtype, "planned cfg%d %s" % (cfg, mode))


@pytest.mark.parametrize("cfg", [3, 4])
def test_sgmv_exact_integer_config_shapes(cfg):
    # full token counts (8192 / 4608), every row bit-exact, fused and split
    # (split: v exact too), split == fused bit for bit
    wl = W.make_workload(cfg, exact=True)
    b = W.make_batch(wl, 0, zero_y0=False)
    used = sorted(set(b.ids.tolist()))
    log("[case] exact sgmv cfg=%d tokens=%d adapters=%d" % (cfg, len(b.ids), len(used)))
    sp = pool_for(("exact", cfg), wl, adapters=used)
    ys, st = run_sgmv(sp, b, [0, 1], wl.dtype, "fused")
    assert st["n_mfma_items"] > 0
    refs = {}
    for s in range(2):
        refs[s] = reference(wl, b, s, wl.dtype, return_v=True)
        exact_compare(ys[s], refs[s][0], wl.dtype, "exact cfg%d s%d" % (cfg, s))
    ys2, _, vs2 = run_sgmv(sp, b, [0, 1], wl.dtype, "split", return_v=True)
    for s in range(2):
        assert ys2[s].tobytes() == ys[s].tobytes()
        assert np.array_equal(vs2[s].astype(np.float64), refs[s][1]), "exact cfg%d s%d v" % (cfg, s)

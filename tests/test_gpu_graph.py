"""The compute entry points under HIP graph capture, through the C ABI.

They allocate nothing and never wait on the host (planned launch shapes are
prepared and the workspace is the caller's), so a stream capture can record
them.  Each graph is replayed several times, with eager work and a host
synchronisation between replays, y reset to y0 before each; every replay must
give the bits of the eager call, which itself matches the fp64 oracle.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import gather_lora_matmul_amd as L  # noqa: E402
import workloads as W  # noqa: E402
from gather_lora_matmul_amd.synthetic import SyntheticPool, from_device, prepare_shapes, to_device  # noqa: E402

from gpu_helpers import check_all, ids_tensor, log  # noqa: E402


def _replay_and_compare(launch, ys, y0s, eager, label, replays=4):
    g = torch.cuda.CUDAGraph()
    for y, y0 in zip(ys, y0s):
        y.copy_(y0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        launch()
    for k in range(replays):
        for y, y0 in zip(ys, y0s):
            y.copy_(y0)
        g.replay()
        junk = torch.randn(4096, device="cuda")
        junk = (junk * 2).sum()  # eager work of the program between replays
        torch.cuda.synchronize()
        for j, (y, e) in enumerate(zip(ys, eager)):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16)), "%s replay %d slice %d" % (label, k, j)


def test_graph_bgmv_apply_with_shared_x():
    wl = W.make_workload(1)
    b = W.make_batch(wl, 0)
    b.x[1] = b.x[0]
    b.x[2] = b.x[0]
    used = sorted(set(int(a) for a in b.ids if a >= 0))
    log("[case] graph capture: lora_bgmv_apply, 64 tokens, q/k/v sharing x")
    sp = SyntheticPool(wl, adapters=used)
    try:
        ids = ids_tensor(b.ids)
        x0 = to_device(b.x[0], wl.act_dtype)
        xs = [x0, x0, x0, to_device(b.x[3], wl.act_dtype)]
        y0s = [to_device(b.y0[s], wl.act_dtype) for s in range(4)]
        ys = [y.clone() for y in y0s]
        io = [(s, xs[s], ys[s], 1 if s < 3 else 0) for s in range(4)]
        ydt = W.DTYPE_CODE[wl.act_dtype]
        call = L.prepare_bgmv_apply(sp.handle, io, ids, ydt)
        call(torch.cuda.current_stream().cuda_stream)  # eager
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        check_all(wl, b, {s: from_device(eager[s], wl.act_dtype) for s in range(4)}, {}, [0, 1, 2, 3],
                  wl.act_dtype, "graph bgmv eager")
        _replay_and_compare(lambda: call(torch.cuda.current_stream().cuda_stream), ys, y0s, eager,
                            "bgmv")
    finally:
        torch.cuda.synchronize()
        sp.close()


def test_graph_planned_apply_mfma_and_short_items():
    # MFMA tiles (two launches, partial tiles in the workspace) and short items
    # in one plan; A rows over two pages
    ids = np.array([0] * 150 + [1] * 65 + [2] * 7 + [3] * 1 + [4] * 40 + [-1] * 3, np.int32)
    np.random.default_rng(7).shuffle(ids)
    wl = W.small_workload("bf16", 2304, 1000, [128, 16, 64, 5, 96], 2048, n_slices=2, seed=31)
    b = W.custom_batch(wl, ids, zero_y0=False)
    log("[case] graph capture: lora_apply, %d tokens, MFMA tiles and short items" % len(ids))
    sp = SyntheticPool(wl)
    plan = L.lora_plan_create(sp.handle, len(ids))
    try:
        L.lora_plan_build(plan, ids, l_long=16)
        st = L.lora_plan_get_stats(plan)
        assert st["n_mfma_items"] > 0 and st["n_items"] > st["n_mfma_items"], st
        ws = prepare_shapes(plan, [[0, 1]])
        xs = [to_device(b.x[s], "bf16") for s in range(2)]
        y0s = [to_device(b.y0[s], "bf16") for s in range(2)]
        ys = [y.clone() for y in y0s]
        io = [(s, xs[s], ys[s]) for s in range(2)]
        call = L.prepare_apply(sp.handle, plan, io, L.LORA_BF16, workspace=ws)
        call(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        check_all(wl, b, {s: from_device(eager[s], "bf16") for s in range(2)}, {}, [0, 1], "bf16",
                  "graph apply eager")
        _replay_and_compare(lambda: call(torch.cuda.current_stream().cuda_stream), ys, y0s, eager,
                            "apply")
    finally:
        torch.cuda.synchronize()
        L.lora_plan_destroy(plan)
        sp.close()


def test_graph_device_planned_decode():
    # the device planner, then the MFMA launches, all from the workspace: the
    # captured graph replays the whole sequence; the ids are changed between
    # replays (the graph reads them at replay time), and every replay gives the
    # bits of an eager call on the same ids
    wl = W.small_workload("bf16", 1024, 1000, [8, 40, 16, 64, 24], 1024, n_slices=2, seed=33)
    rng = np.random.default_rng(5)
    ids_a = rng.integers(-1, 5, 200).astype(np.int32)
    ids_b = rng.integers(0, 5, 200).astype(np.int32)
    ids_b[:90] = 3
    log("[case] graph capture: lora_bgmv_apply_planned, 200 tokens, ids changed between replays")
    sp = SyntheticPool(wl)
    try:
        ba = W.custom_batch(wl, ids_a, zero_y0=False)
        bb = W.custom_batch(wl, ids_b, zero_y0=False)
        ids = ids_tensor(ids_a)
        xs = [to_device(ba.x[s], "bf16") for s in range(2)]
        y0s = [to_device(ba.y0[s], "bf16") for s in range(2)]
        ys = [y.clone() for y in y0s]
        ws = torch.empty(L.lora_bgmv_planned_workspace_size(sp.handle, [0, 1], 200), dtype=torch.uint8,
                         device="cuda")
        call = L.prepare_bgmv_apply_planned(sp.handle, [(s, xs[s], ys[s]) for s in range(2)], ids,
                                            L.LORA_BF16, ws)
        eager = {}
        for key, idv in (("a", ids_a), ("b", ids_b)):
            ids.copy_(torch.from_numpy(idv))
            for y, y0 in zip(ys, y0s):
                y.copy_(y0)
            call(torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            eager[key] = [y.clone() for y in ys]
        bref = W.Batch(ids=ids_b, x=ba.x, y0=ba.y0)
        check_all(wl, bref, {s: from_device(eager["b"][s], "bf16") for s in range(2)}, {}, [0, 1],
                  "bf16", "graph devplan eager")
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            call(torch.cuda.current_stream().cuda_stream)
        for k in range(6):
            key = "ab"[k % 2]
            ids.copy_(torch.from_numpy(ids_a if key == "a" else ids_b))
            for y, y0 in zip(ys, y0s):
                y.copy_(y0)
            g.replay()
            junk = (torch.randn(4096, device="cuda") * 2).sum()  # eager work between replays
            torch.cuda.synchronize()
            for j in range(2):
                assert torch.equal(ys[j].view(torch.int16), eager[key][j].view(torch.int16)), \
                    "replay %d (ids %s) slice %d" % (k, key, j)
        del bb, junk
    finally:
        torch.cuda.synchronize()
        sp.close()

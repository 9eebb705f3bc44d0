"""lora_apply_noalloc: the planned fused apply with the library's static
scratch as its partial-tile workspace (for callers that cannot allocate).

GPU: its output equals lora_apply's (same kernels, same summation order: bit
for bit) and the oracle's, on two calls in a row, the second with a smaller
batch.  CPU: a launch shape whose partial tiles exceed the scratch is refused.
"""
import numpy as np
import pytest

import gather_lora_matmul_amd as L
import workloads as W

SCRATCH_BYTES = 16 << 20


def test_noalloc_refuses_shapes_beyond_the_scratch():
    # rank-128 tiles over eight slices: the partial tiles need more than 16 MiB
    from gather_lora_matmul_amd.synthetic import SyntheticPool
    wl = W.small_workload("bf16", 2048, 256, [128], 2048, n_slices=8)
    ids = np.zeros(64 * 120, np.int32)
    with SyntheticPool(wl, host_only=True, poison=False) as sp:
        plan = L.lora_plan_create(sp.handle, len(ids))
        try:
            L.lora_plan_build(plan, ids, stream=0)
            L.lora_plan_prepare(plan, list(range(8)), stream=0)
            need = L.lora_workspace_size(plan, list(range(8)))
            assert need > SCRATCH_BYTES
            fake = 1 << 20  # never dereferenced: the call fails on the host
            io = (L.Io * 8)(*[L.Io(s, 0, fake, fake) for s in range(8)])
            st = L.lib().lora_apply_noalloc(sp.handle, plan, 8, io, L.LORA_BF16, None)
            assert st == -1 and "static scratch" in L.lora_last_error()
            L.lora_plan_prepare(plan, [0], stream=0)
            assert L.lora_workspace_size(plan, [0]) <= SCRATCH_BYTES
            io1 = (L.Io * 1)(L.Io(0, 0, fake, fake))
            st = L.lib().lora_apply_noalloc(sp.handle, plan, 1, io1, L.LORA_BF16, None)
            assert st == -5  # fits: refused only because a host-only pool runs nothing
        finally:
            L.lora_plan_destroy(plan)


@pytest.mark.gpu
def test_noalloc_matches_lora_apply_twice():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gather_lora_matmul_amd.synthetic import SyntheticPool, prepare_shapes, to_device
    from gpu_helpers import Guarded, compare, log, reference
    wl = W.small_workload("bf16", 512, 1000, [16, 64, 5, 128, 33], 512, n_slices=2, seed=61)
    big = np.array([0] * 150 + [1] * 65 + [2] * 7 + [3] * 90 + [4] * 40 + [-1] * 3, np.int32)
    small = np.array([3] * 20 + [1] * 17 + [0, 2, 4] * 3 + [-1], np.int32)
    rng = np.random.default_rng(8)
    with SyntheticPool(wl) as sp:
        for k, ids in enumerate((big, small)):
            ids = ids.copy()
            rng.shuffle(ids)
            log("[case] noalloc call %d, %d tokens" % (k, len(ids)))
            b = W.custom_batch(wl, ids, index=k, zero_y0=(k == 0))
            plan = L.lora_plan_create(sp.handle, len(ids))
            try:
                L.lora_plan_build(plan, ids)
                ws = prepare_shapes(plan, [[0, 1]])
                assert L.lora_plan_get_stats(plan)["n_mfma_items"] > 0
                xs = [to_device(b.x[s], "bf16") for s in range(2)]
                y_ws = [Guarded(b.y0[s], "bf16") for s in range(2)]
                y_na = [Guarded(b.y0[s], "bf16") for s in range(2)]
                L.lora_apply(sp.handle, plan, [(s, xs[s], y_ws[s].view) for s in range(2)],
                             L.LORA_BF16, workspace=ws)
                L.lora_apply_noalloc(sp.handle, plan, [(s, xs[s], y_na[s].view) for s in range(2)],
                                     L.LORA_BF16)
                torch.cuda.synchronize()
                for s in range(2):
                    got, want = y_na[s].host(), y_ws[s].host()
                    assert got.tobytes() == want.tobytes(), "call %d slice %d differs" % (k, s)
                    compare(got, reference(wl, b, s, "bf16"), "bf16", "noalloc call %d s%d" % (k, s))
            finally:
                L.lora_plan_destroy(plan)

"""GPU parity of FP8 E4M3 adapter pages (per-rank scales, 16-bit activations)
against the fp64 oracle, through the C ABI.

Inputs come from `workloads` (seeded); expected values only from `oracle`.
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
from gather_lora_matmul_amd.synthetic import SyntheticPool, to_device  # noqa: E402

from gpu_helpers import (check_all, exact_compare, ids_tensor, log, reference, run_bgmv,  # noqa: E402
                         run_sgmv)

_POOLS = {}


def pool_for(key, wl, adapters=None):
    if key not in _POOLS:
        log("[setup] fp8 pool %s" % (key,))
        _POOLS[key] = SyntheticPool(wl, adapters=adapters)
    return _POOLS[key]


@pytest.fixture(scope="module", autouse=True)
def _cleanup():
    yield
    for p in _POOLS.values():
        p.close()
    _POOLS.clear()
    torch.cuda.synchronize()


def test_decoder_all_e4m3_codes_and_16bit_patterns():
    # the kernels' own decoders (lora_debug_decode) against the oracle's, bit
    # for bit: all 256 E4M3 codes (NaN codes stay NaN), and random 16-bit and
    # fp32 patterns including subnormals
    log("[case] device decoders")
    codes = np.arange(256, dtype=np.uint8)
    src = to_device(codes, "e4m3")
    dst = torch.full((256,), 7.0, dtype=torch.float32, device="cuda")
    L.lora_debug_decode(L.LORA_FP8_E4M3, src, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().astype(np.float64)
    want = oracle.decode(codes, "e4m3")
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(want[ok]))
    rng = np.random.default_rng(0)
    for dt, code in (("f16", L.LORA_F16), ("bf16", L.LORA_BF16)):
        bits = rng.integers(0, 1 << 16, size=4096).astype(np.uint16)
        bits = bits[np.isfinite(oracle.decode(bits, dt))]
        bits = bits[: len(bits) // 8 * 8]
        dst = torch.zeros(len(bits), dtype=torch.float32, device="cuda")
        L.lora_debug_decode(code, to_device(bits, dt), dst)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(dst.cpu().numpy().astype(np.float64), oracle.decode(bits, dt))


def test_fp8_gather_bit_exact():
    wl = W.small_workload("e4m3", 272, 200, [5, 16, 40, 128], 256, n_slices=2, act_dtype="bf16")
    log("[case] fp8 gather")
    sp = pool_for("gather", wl)
    for s in range(2):
        for a in range(4):
            r = int(wl.ranks[a])
            A = torch.zeros((r, 272), dtype=torch.uint8, device="cuda")
            B = torch.zeros((200, r), dtype=torch.uint8, device="cuda")
            L.lora_debug_gather(sp.handle, s, a, A, B)
            torch.cuda.synchronize()
            A0, B0 = wl.weights(a, s)
            assert A.cpu().numpy().tobytes() == A0.tobytes()
            assert B.cpu().numpy().tobytes() == B0.tobytes()
            sa, sb = L.lora_pool_export_scales(sp.handle, a, s, r)
            qa, qb = wl.qscales(a, s)
            assert sa.tobytes() == qa.tobytes() and sb.tobytes() == qb.tobytes()


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_fp8_llama7b_decode_full(mode):
    # the quantised Llama-7B decode batch: 64 tokens x q/k/v/o, every row (and v)
    wl = W.make_workload(5)
    b = W.make_batch(wl, 0)
    log("[case] fp8 llama7b decode full mode=%s" % mode)
    sp = pool_for("cfg5", wl)
    ys, vs = run_bgmv(sp, b, [0, 1, 2, 3], wl.act_dtype, mode, return_v=True)
    check_all(wl, b, ys, vs, [0, 1, 2, 3], wl.act_dtype, "fp8 cfg5 %s" % mode)
    # fp32 y on a random y0 (delta gated too)
    b32 = W.make_batch(wl, 1, y_dtype="f32", zero_y0=False)
    ys, vs = run_bgmv(sp, b32, [2], "f32", mode, return_v=True)
    check_all(wl, b32, ys, vs, [2], "f32", "fp8 cfg5 f32 %s" % mode)


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_fp8_exact_integer_bit_exact(mode):
    # codes of -1, 0, 1 with power-of-two scales: every partial sum is exact,
    # so y (and v) must equal the oracle bit for bit
    wl = W.make_workload(5, exact=True)
    b = W.make_batch(wl, 0, zero_y0=False)
    used = sorted(set(b.ids.tolist()))
    log("[case] fp8 exact mode=%s adapters=%d" % (mode, len(used)))
    sp = pool_for(("exact", 5), wl, adapters=used)
    ys, vs = run_bgmv(sp, b, [0, 1, 2, 3], wl.act_dtype, mode, return_v=True)
    for s in range(4):
        y_ref, v_ref = reference(wl, b, s, wl.act_dtype, return_v=True)
        exact_compare(ys[s], y_ref, wl.act_dtype, "fp8 exact s%d" % s)
        if s in vs:
            assert np.array_equal(vs[s].astype(np.float64), v_ref), "fp8 exact s%d v" % s


SMALL = [
    # d_in, d_out, ranks, P, act, ids
    (512, 520, [16, 64, 5, 128], 256, "bf16", [0] * 70 + [1] * 17 + [2] * 3 + [3] * 30 + [-1] * 5),
    (272, 264, [8, 40, 1], 256, "f16", [1] * 33 + [0, 2, 1, 0] * 9 + [2] * 16),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("mode", ["split", "fused"])
@pytest.mark.parametrize("entry", ["bgmv", "planned"])
def test_fp8_small(case, mode, entry):
    # odd ranks (r_s padding of the one-byte B rows), A rows over two pages,
    # d_out not a multiple of a page's B rows; planned batches run as short
    # VALU items (no MFMA tiles on FP8 pages)
    d_in, d_out, ranks, P, act, ids = SMALL[case]
    log("[case] fp8 small %d %s %s" % (case, entry, mode))
    wl = W.small_workload("e4m3", d_in, d_out, ranks, P, n_slices=2, seed=80 + case, act_dtype=act)
    ids = np.array(ids, np.int32)
    np.random.default_rng(case).shuffle(ids)
    b = W.custom_batch(wl, ids, zero_y0=True)
    sp = pool_for(("small", case), wl)
    if entry == "bgmv":
        ys, vs = run_bgmv(sp, b, [0, 1], act, mode, return_v=True)
    else:
        ys, st, vs = run_sgmv(sp, b, [0, 1], act, mode, return_v=True)
        assert st["n_mfma_items"] == 0 and st["n_items"] > 0
    check_all(wl, b, ys, vs, [0, 1], act, "fp8 small %d %s %s" % (case, entry, mode))


def test_fp8_out_of_table_ids_skipped():
    wl = W.small_workload("e4m3", 272, 264, [8, 40, 1], 256, n_slices=2, seed=81, act_dtype="f16")
    sp = pool_for(("small", 1), wl)
    ids = np.array([0, 3, -1, 1, 2 ** 31 - 1, 2], np.int32)
    b = W.custom_batch(wl, ids, zero_y0=False)
    log("[case] fp8 skipped ids")
    ys = run_bgmv(sp, b, [0, 1], "f16", "fused")
    skip = (ids < 0) | (ids >= 3)
    ref_b = W.Batch(ids=np.where(skip, -1, ids).astype(np.int32), x=b.x, y0=b.y0)
    check_all(wl, ref_b, ys, {}, [0, 1], "f16", "fp8 skipped ids")
    for s in (0, 1):
        assert ys[s][skip].tobytes() == b.y0[s][skip].tobytes()
    assert ids_tensor(ids).dtype == torch.int32

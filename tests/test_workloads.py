"""The seeded input generators: determinism and the stated distributions."""
import numpy as np
import pytest

import workloads as W


def test_same_seed_same_bytes():
    a = W.make_workload(0)
    b = W.make_workload(0)
    for ad in range(4):
        for x, y in zip(a.weights(ad, 0), b.weights(ad, 0)):
            assert x.tobytes() == y.tobytes()
    ba, bb = W.make_batch(a, 3), W.make_batch(b, 3)
    assert ba.ids.tobytes() == bb.ids.tobytes()
    assert ba.x[0].tobytes() == bb.x[0].tobytes()


def test_tiny_config_matches_description():
    wl = W.make_workload(0)
    assert wl.ranks.tolist() == [4, 8, 8, 16]
    assert np.allclose(wl.scales, [4, 2, 2, 1])
    b = W.make_batch(wl, 0)
    assert b.ids.shape == (8,) and b.ids.min() >= 0 and b.ids.max() < 4
    A, B = wl.weights(3, 0)
    assert A.shape == (16, 256) and B.shape == (256, 16) and A.dtype == np.float32
    assert abs(float(np.std(np.concatenate([A.ravel(), B.ravel()]))) - 0.02) < 0.002


def test_quantize_bf16_rne():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-40])
    q = W.dequantize(W.quantize(v, "bf16"), "bf16")
    assert q[0] == 1.0 and q[1] == 1.0 and q[2] == 1.0 + 2 ** -6 and q[3] == -2.5


def test_lognormal_lengths_total():
    rng = np.random.default_rng(0)
    lens = W.lognormal_lengths(rng, 32, 256, 8192)
    assert lens.sum() == 8192 and lens.min() >= 1 and lens.shape == (32,)


def test_zipf_concentration():
    rng = np.random.default_rng(1)
    perm = np.arange(2000)
    ids = W.zipf_ids(rng, 200000, 2000, 1.0, perm)
    top = np.mean(ids == 0)
    # H_2000(1) ~ 8.18 -> p(top) ~ 0.122
    assert abs(top - 1 / sum(1 / k for k in range(1, 2001))) < 0.01


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_configs_shapes(cfg):
    wl = W.make_workload(cfg)
    b = W.make_batch(wl, 0, with_x=False)
    if cfg == 1:
        assert wl.dtype == "f16" and set(wl.ranks.tolist()) == {16} and b.ids.shape == (64,)
        assert wl.slices == [(4096, 4096)] * 4
    if cfg == 2:
        assert set(wl.ranks.tolist()) <= {8, 16, 32, 64} and b.ids.shape == (256,)
        assert wl.slices == [(4096, 4096), (4096, 11008)]
    if cfg == 3:
        assert b.ids.shape == (8192,) and b.seg_lengths.sum() == 8192
        # equal adapters are contiguous (requests sorted by adapter)
        change = np.flatnonzero(np.diff(b.ids)) + 1
        runs = np.split(b.ids, change)
        assert len(set(int(r[0]) for r in runs)) == len(runs)


def test_mixed_config_layout():
    wl = W.make_workload(4)
    assert wl.ranks.min() >= 8 and wl.ranks.max() <= 128
    b = W.make_batch(wl, 0, with_x=False)
    assert b.ids.shape == (4608,) and b.n_decode == 512 and b.seg_lengths.sum() == 4096
    A, B = wl.weights(int(b.ids[0]), 1)
    assert B.shape == (28672, int(wl.ranks[b.ids[0]]))


def test_exact_mode_values():
    wl = W.small_workload("bf16", 32, 16, [3, 9], 32, exact=True)
    A, B = wl.weights(1, 0)
    assert set(np.unique(W.dequantize(A, "bf16")).tolist()) <= {-1.0, 0.0, 1.0}
    assert all(float(s) == 2.0 ** -np.floor(np.log2(r)) for s, r in zip(wl.scales, wl.ranks))


def test_e4m3_generator_matches_torch_conversion():
    # the input quantiser (RNE, saturating) and decoder of the generators agree
    # with torch's float8_e4m3fn conversions
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 100, 100000), rng.normal(0, 0.01, 10000),
                        [448.0, 449.0, 464.0, 1e9, -1e9, 0.0, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -9]])
    q = W.quantize_e4m3(x)
    qt = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, qt)
    codes = np.arange(256, dtype=np.uint8)
    d = W.dequantize(codes, "e4m3")
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(d), np.isnan(ref))
    np.testing.assert_array_equal(d[~np.isnan(d)], ref[~np.isnan(ref)])


def test_quantised_workload_shapes():
    wl = W.make_workload(5)
    assert wl.dtype == "e4m3" and wl.act_dtype == "f16" and wl.quantized
    A, B = wl.weights(3, 1)
    sa, sb = wl.qscales(3, 1)
    assert A.dtype == np.uint8 and A.shape == (16, 4096) and B.shape == (4096, 16)
    assert sa.dtype == np.float32 and sa.shape == (16,) and sb.shape == (16,)
    w = sa[:, None].astype(np.float64) * W.dequantize(A, "e4m3")
    assert 0.012 < w.std() < 0.03 and np.all(np.isfinite(w))
    b = W.make_batch(wl, 0)
    assert b.x[0].dtype == np.uint16 and len(b.ids) == 64

"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle with something independent: a value the
method's definition gives by hand, a closed form, a textbook special case that a
library routine computes, exact integer arithmetic, or exact rationals.  Chosen
so that a dropped term, a wrong sign or index, a transposed operand or a
misplaced scale fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dense(wl, a, s=0):
    A, B = wl.weights(a, s)
    return W.dequantize(A, wl.dtype), W.dequantize(B, wl.dtype)


# --- decoders and rounding --------------------------------------------------
def test_decode_matches_ieee_views():
    rng = np.random.default_rng(0)
    h = rng.integers(0, 1 << 16, size=20000, dtype=np.uint64).astype(np.uint16)
    finite = np.isfinite(h.view(np.float16))
    got = oracle.decode(h, "f16")
    np.testing.assert_array_equal(got[finite], h.view(np.float16)[finite].astype(np.float64))
    ref = h.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    b = h
    fb = (b.astype(np.uint32) << 16).view(np.float32)
    ok = np.isfinite(fb)
    np.testing.assert_array_equal(oracle.decode(b, "bf16")[ok], fb[ok].astype(np.float64))
    # every fp16 subnormal decodes to m * 2^-24
    sub = np.arange(1, 1024, dtype=np.uint16)
    np.testing.assert_array_equal(oracle.decode(sub, "f16"), sub.astype(np.float64) * 2.0 ** -24)


def _rne_exact(v: float, p: int, emin: int, emax: int) -> float:
    """Round-to-nearest-even with exact rationals (textbook definition)."""
    if v == 0:
        return v
    fv = Fraction(v)
    a = abs(fv)
    e = math.floor(math.log2(a)) if a != 0 else emin
    # fix float-log rounding at powers of two
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - (p - 1))
    t = a / q
    fl = math.floor(t)
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    if r >= Fraction(2) ** (emax + 1):
        return math.copysign(math.inf, v)
    return math.copysign(float(r), v)


@pytest.mark.parametrize("dtype,p,emin,emax", [("bf16", 8, -126, 127), ("f16", 11, -14, 15),
                                                ("f32", 24, -126, 127)])
def test_round_matches_exact_rne(dtype, p, emin, emax):
    rng = np.random.default_rng(1)
    vals = list(rng.normal(0, 1, 300)) + list(rng.normal(0, 1e-6, 100)) + \
        list(rng.normal(0, 2.0 ** emin, 100))
    # exact ties: midpoints between neighbours, both parities
    for k in range(1, 40):
        base = 1.0 + k * 2.0 ** (1 - p)
        vals += [base + 2.0 ** -p, -(base + 2.0 ** -p)]
    big = (2 - 2.0 ** (1 - p)) * 2.0 ** emax
    vals += [big, big * (1 + 2.0 ** -(p + 1)), 2.0 ** (emax + 1), -big * 1.0000001]
    vals = np.array(vals, np.float64)
    got = oracle.decode(oracle.round_to(vals, dtype), dtype)
    want = np.array([_rne_exact(float(v), p, emin, emax) for v in vals])
    np.testing.assert_array_equal(got, want)


def test_round_f16_agrees_with_numpy():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e-5, 5000), rng.normal(0, 3e4, 500)])
    with np.errstate(over="ignore"):
        ref16 = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.round_to(v, "f16"), ref16)
    np.testing.assert_array_equal(oracle.round_to(v, "f32"), v.astype(np.float32))


# --- the worked example of the index-vector diagram -------------------------
def _golden():
    with open(os.path.join(GOLDEN, "index_vector_example.json")) as f:
        return json.load(f)


def test_index_vector_example_by_hand():
    g = _golden()
    na = g["n_adapters"]
    ranks = np.zeros(na, np.int32)
    scales = np.zeros(na, np.float32)
    weights = {}
    for k, ad in g["adapters"].items():
        a = int(k)
        ranks[a] = ad["rank"]
        scales[a] = ad["scale"]
        weights[a] = (np.array(ad["A"], np.float32), np.array(ad["B"], np.float32))
    y = oracle.lora_apply(np.array(g["x"], np.float32), np.array(g["ids"], np.int32), ranks,
                          scales, weights, np.array(g["y0"], np.float32), "f32", "f32")
    np.testing.assert_array_equal(y, np.array(g["y_expected"], np.float64))


# --- P1: scale 0 leaves y untouched; P2: id -1 leaves y untouched ---------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_scale_zero_and_negative_id_leave_y(dtype):
    wl = W.small_workload(dtype, 64, 48, [3, 8, 5], 64, scales=[0.0, 0.0, 0.0])
    b = W.custom_batch(wl, [0, 1, 2, -1, 1, 0])
    y = oracle.workload_reference(wl, b, 0)
    np.testing.assert_array_equal(y, W.dequantize(b.y0[0], dtype))
    wl2 = W.small_workload(dtype, 64, 48, [3, 8, 5], 64)
    b2 = W.custom_batch(wl2, [-1, -1, 2, -1])
    y2 = oracle.workload_reference(wl2, b2, 0)
    y0 = W.dequantize(b2.y0[0], dtype)
    np.testing.assert_array_equal(y2[[0, 1, 3]], y0[[0, 1, 3]])
    assert np.abs(y2[2] - y0[2]).max() > 0


# --- P3: all tokens on one adapter = a dense two-GEMM product (BLAS) -------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_adapter_equals_two_gemms(dtype):
    wl = W.small_workload(dtype, 96, 80, [7], 96)
    b = W.custom_batch(wl, [0] * 11)
    y = oracle.workload_reference(wl, b, 0)
    A, B = _dense(wl, 0)
    X = W.dequantize(b.x[0], dtype)
    Y0 = W.dequantize(b.y0[0], dtype)
    ref = Y0 + float(wl.scales[0]) * ((X @ A.T) @ B.T)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    # the scale sits outside the product exactly once
    assert np.abs(y - (Y0 + (X @ A.T) @ B.T)).max() > 1e-6


# --- P4: rank-1 adapters -> closed-form outer product -----------------------
def test_rank1_closed_form():
    rng = np.random.default_rng(3)
    d_in, d_out, n = 40, 24, 9
    a = rng.integers(-3, 4, size=d_in).astype(np.float32)
    bb = rng.integers(-3, 4, size=d_out).astype(np.float32)
    X = rng.integers(-5, 6, size=(n, d_in)).astype(np.float32)
    Y0 = rng.integers(-5, 6, size=(n, d_out)).astype(np.float32)
    s = np.float32(0.25)
    y = oracle.lora_apply(X, np.zeros(n, np.int32), np.array([1], np.int32), np.array([s]),
                          {0: (a[None, :], bb[:, None])}, Y0, "f32", "f32")
    for i in range(n):
        dot = sum(int(a[j]) * int(X[i, j]) for j in range(d_in))
        want = [Fraction(int(Y0[i, m])) + Fraction(1, 4) * dot * int(bb[m]) for m in range(d_out)]
        assert [Fraction(v) for v in y[i]] == want


# --- P5: exact-integer inputs -> exact result in any order ------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_exact_integer_mode(dtype):
    wl = W.small_workload(dtype, 128, 72, [8, 5, 16, 1], 128, exact=True)
    b = W.custom_batch(wl, [3, 0, 2, 2, -1, 1, 0, 3])
    y = oracle.workload_reference(wl, b, 0)
    X = W.dequantize(b.x[0], dtype).astype(np.int64)
    Y0 = W.dequantize(b.y0[0], dtype).astype(np.int64)
    for i, a in enumerate(b.ids.tolist()):
        if a < 0:
            np.testing.assert_array_equal(y[i], Y0[i])
            continue
        A, B = _dense(wl, a)
        v = A.astype(np.int64) @ X[i]
        d = B.astype(np.int64) @ v
        want = [Fraction(int(Y0[i, m])) + Fraction(float(wl.scales[a])) * int(d[m])
                for m in range(d.shape[0])]
        assert [Fraction(t) for t in y[i]] == want


# --- P6: brute force with exact rationals, the other association order ------
def test_brute_force_rationals_within_bound():
    wl = W.small_workload("f32", 8, 6, [4, 3, 2], 8, seed=11)
    b = W.custom_batch(wl, [1, 0, 2, 1, -1, 0])
    y = oracle.workload_reference(wl, b, 0)
    X = W.dequantize(b.x[0], "f32")
    Y0 = W.dequantize(b.y0[0], "f32")
    u = 2.0 ** -53
    for i, a in enumerate(b.ids.tolist()):
        if a < 0:
            continue
        A, B = _dense(wl, a)
        r = int(wl.ranks[a])
        s = Fraction(float(wl.scales[a]))
        # materialise Delta W = s B A exactly, then apply it
        dW = [[s * sum(Fraction(B[m, k]) * Fraction(A[k, j]) for k in range(r))
               for j in range(8)] for m in range(6)]
        for m in range(6):
            exact = Fraction(Y0[i, m]) + sum(dW[m][j] * Fraction(X[i, j]) for j in range(8))
            mag = abs(Y0[i, m]) + float(s) * sum(
                abs(B[m, k]) * sum(abs(A[k, j] * X[i, j]) for j in range(8)) for k in range(r))
            n_ops = 8 + r + 2
            bound = (n_ops * u / (1 - n_ops * u)) * mag
            assert abs(Fraction(y[i, m]) - exact) <= Fraction(bound) + Fraction(1, 10 ** 300)


# --- P10: bilinearity in x ----------------------------------------------------
def test_linearity_in_x():
    wl = W.small_workload("f32", 32, 20, [6, 9], 32, seed=13)
    rng = np.random.default_rng(4)
    n = 5
    ids = np.array([0, 1, 1, 0, 1], np.int32)
    # dyadic values with few bits so x1 + x2 is exact in fp32
    x1 = (rng.integers(-64, 64, size=(n, 32)) / 16.0).astype(np.float32)
    x2 = (rng.integers(-64, 64, size=(n, 32)) / 16.0).astype(np.float32)
    y0 = np.zeros((n, 20), np.float32)
    wts = {a: wl.weights(a, 0) for a in (0, 1)}
    f = lambda x: oracle.lora_apply(x, ids, wl.ranks, wl.scales, wts, y0, "f32", "f32")
    lhs = f(x1 + x2)
    rhs = f(x1) + f(x2)
    assert np.abs(lhs - rhs).max() <= 1e-12 * np.abs(lhs).max()


def test_per_token_independence_and_permutation():
    wl = W.small_workload("bf16", 64, 40, [4, 12, 7], 64, seed=17)
    b = W.custom_batch(wl, [2, 0, 1, 2, 0, -1, 1])
    y = oracle.workload_reference(wl, b, 0)
    perm = np.array([6, 3, 0, 5, 1, 4, 2])
    b2 = W.Batch(ids=b.ids[perm], x=[b.x[0][perm]], y0=[b.y0[0][perm]])
    y2 = oracle.workload_reference(wl, b2, 0)
    np.testing.assert_array_equal(y2, y[perm])


def test_missing_adapter_fails_loudly():
    wl = W.small_workload("f32", 16, 16, [2, 2], 16)
    b = W.custom_batch(wl, [0, 1])
    with pytest.raises(KeyError):
        oracle.lora_apply(b.x[0], b.ids, wl.ranks, wl.scales, {0: wl.weights(0, 0)}, b.y0[0],
                          "f32", "f32")


def test_v_output_is_shrink():
    wl = W.small_workload("f16", 48, 16, [5, 3], 48, seed=19)
    b = W.custom_batch(wl, [1, 0, -1])
    _, v = oracle.workload_reference(wl, b, 0, return_v=True)
    X = W.dequantize(b.x[0], "f16")
    for i, a in enumerate(b.ids.tolist()):
        if a < 0:
            assert np.all(v[i] == 0)
            continue
        A, _ = _dense(wl, a)
        r = int(wl.ranks[a])
        np.testing.assert_allclose(v[i, :r], A @ X[i], rtol=1e-12, atol=1e-14)
        assert np.all(v[i, r:] == 0)


# --- the page walker against a hand-laid pool image -------------------------
@pytest.mark.parametrize("dtype,rank,P,d_in,d_out", [("bf16", 5, 32, 48, 40), ("f32", 3, 16, 16, 23),
                                                     ("f16", 16, 64, 64, 100)])
def test_walker_reads_documented_layout(dtype, rank, P, d_in, d_out):
    rng = np.random.default_rng(5)
    sd = np.float32 if dtype == "f32" else np.uint16
    elt = 4 if dtype == "f32" else 2
    per16 = 16 // elt
    rs = -(-rank // per16) * per16
    npa = -(-d_in // P)
    rpp = P // rs
    npb = -(-d_out // rpp)
    n_pages = rank * npa + npb + 7
    pages = rng.permutation(n_pages)[: rank * npa + npb].astype(np.int32)
    a_pages, b_pages = pages[: rank * npa], pages[rank * npa:]
    pool = np.full(n_pages * P, 0x7FC0 if sd is np.uint16 else np.nan, sd)
    A = rng.integers(1, 1000, size=(rank, d_in)).astype(sd)
    B = rng.integers(1, 1000, size=(d_out, rank)).astype(sd)
    for k in range(rank):
        for j in range(d_in):
            pool[a_pages[k * npa + j // P] * P + j % P] = A[k, j]
    for m in range(d_out):
        base = b_pages[m // rpp] * P + (m % rpp) * rs
        pool[base: base + rs] = 0
        pool[base: base + rank] = B[m]
    A2, B2 = oracle.walk_adapter(pool, dtype, P, d_in, d_out, rank, a_pages, b_pages)
    np.testing.assert_array_equal(A2, A)
    np.testing.assert_array_equal(B2, B)
    if rs > rank:
        pool[b_pages[0] * P + rank] = 1
        with pytest.raises(ValueError):
            oracle.walk_adapter(pool, dtype, P, d_in, d_out, rank, a_pages, b_pages)


# --- quantised adapters: OCP FP8 E4M3 codes with per-row / per-column scales ----
# Values of the format's defining codes (sign, 4 exponent bits with bias 7, 3
# mantissa bits; subnormals m * 2^-9; no infinities; S.1111.111 is NaN).
E4M3_ANCHORS = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2 ** -6,
                0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
                0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}


def test_e4m3_decoder_against_torch_and_the_format():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode(codes, "e4m3")
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    assert int(np.isnan(got).sum()) == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    for c, v in E4M3_ANCHORS.items():
        assert got[c] == v and np.signbit(got[c]) == np.signbit(v), hex(c)
    # monotone over the positive finite codes, symmetric in the sign bit
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)
    np.testing.assert_array_equal(got[0x80:0xFF], -got[:0x7F])


def _quant_dense(wl, a, s=0):
    """Dequantised A, B of a quantised adapter, decoded by torch (independent of
    the oracle) and scaled with numpy."""
    torch = pytest.importorskip("torch")
    A, B = wl.weights(a, s)
    sa, sb = wl.qscales(a, s)
    dec = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()
    return sa.astype(np.float64)[:, None] * dec(A), dec(B) * sb.astype(np.float64)[None, :]


def test_quantised_one_adapter_equals_two_gemms():
    # P3 for quantised adapters: y0 + s (X A^T) B^T with A = diag(sa) A_q, B = B_q diag(sb)
    wl = W.small_workload("e4m3", 96, 80, [7], 96, act_dtype="bf16")
    b = W.custom_batch(wl, [0] * 11)
    y = oracle.workload_reference(wl, b, 0)
    A, B = _quant_dense(wl, 0)
    X = W.dequantize(b.x[0], "bf16")
    Y0 = W.dequantize(b.y0[0], "bf16")
    ref = Y0 + float(wl.scales[0]) * ((X @ A.T) @ B.T)
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    # dropping either scale set, or applying the row scales of A to B, fails
    sa, sb = wl.qscales(0, 0)
    Aq, Bq = A / sa[:, None], B / sb[None, :]
    for wrong in ((Aq, B), (A, Bq), (A, Bq * sa[None, :])):
        bad = Y0 + float(wl.scales[0]) * ((X @ wrong[0].T) @ wrong[1].T)
        assert np.abs(y - bad).max() > 1e-3 * np.abs(ref - Y0).max()


def test_quantised_rank1_closed_form():
    # y_i = y0_i + s * sa * sb * (a_q . x_i) * b_q, exactly
    rng = np.random.default_rng(21)
    d_in, d_out, n = 40, 24, 7
    aq = rng.integers(-3, 4, size=d_in).astype(np.float64)
    bq = rng.integers(-3, 4, size=d_out).astype(np.float64)
    A = W.quantize_e4m3(aq)[None, :]
    B = W.quantize_e4m3(bq)[:, None]
    X = rng.integers(-5, 6, size=(n, d_in)).astype(np.float32)
    Y0 = rng.integers(-5, 6, size=(n, d_out)).astype(np.float32)
    sa, sb, s = np.float32(0.375), np.float32(1.25), np.float32(0.5)
    y = oracle.lora_apply(X, np.zeros(n, np.int32), np.array([1], np.int32), np.array([s]),
                          {0: (A, B, np.array([sa]), np.array([sb]))}, Y0, "e4m3", "f32",
                          x_dtype="f32")
    for i in range(n):
        dot = sum(int(aq[j]) * int(X[i, j]) for j in range(d_in))
        k = Fraction(float(s)) * Fraction(float(sa)) * Fraction(float(sb)) * dot
        want = [Fraction(int(Y0[i, m])) + k * int(bq[m]) for m in range(d_out)]
        assert [Fraction(v) for v in y[i]] == want


def test_quantised_exact_integer_mode():
    wl = W.small_workload("e4m3", 128, 72, [8, 5, 16, 1], 128, exact=True, act_dtype="f16")
    b = W.custom_batch(wl, [3, 0, 2, 2, -1, 1, 0, 3])
    y, v = oracle.workload_reference(wl, b, 0, return_v=True)
    X = W.dequantize(b.x[0], "f16")
    Y0 = W.dequantize(b.y0[0], "f16")
    for i, a in enumerate(b.ids.tolist()):
        if a < 0:
            np.testing.assert_array_equal(y[i], Y0[i])
            continue
        A, B = _quant_dense(wl, a)
        vi = [sum(Fraction(A[k, j]) * Fraction(X[i, j]) for j in range(128)) for k in range(A.shape[0])]
        assert [Fraction(t) for t in v[i, :A.shape[0]]] == vi
        want = [Fraction(Y0[i, m]) + Fraction(float(wl.scales[a])) *
                sum(Fraction(B[m, k]) * vi[k] for k in range(A.shape[0])) for m in range(72)]
        assert [Fraction(t) for t in y[i]] == want


def test_walker_reads_e4m3_layout():
    # one-byte elements: r_s = rank rounded up to 16, floor(P / r_s) B rows per page
    rng = np.random.default_rng(6)
    rank, P, d_in, d_out = 5, 64, 100, 30
    rs, npa = 16, -(-100 // 64)
    rpp = P // rs
    npb = -(-d_out // rpp)
    n_pages = rank * npa + npb + 5
    pages = rng.permutation(n_pages)[: rank * npa + npb].astype(np.int32)
    a_pages, b_pages = pages[: rank * npa], pages[rank * npa:]
    pool = np.full(n_pages * P, 0x7F, np.uint8)
    A = rng.integers(1, 0x7E, size=(rank, d_in)).astype(np.uint8)
    B = rng.integers(1, 0x7E, size=(d_out, rank)).astype(np.uint8)
    for k in range(rank):
        for j in range(d_in):
            pool[a_pages[k * npa + j // P] * P + j % P] = A[k, j]
    for m in range(d_out):
        base = b_pages[m // rpp] * P + (m % rpp) * rs
        pool[base: base + rs] = 0
        pool[base: base + rank] = B[m]
    A2, B2 = oracle.walk_adapter(pool, "e4m3", P, d_in, d_out, rank, a_pages, b_pages)
    np.testing.assert_array_equal(A2, A)
    np.testing.assert_array_equal(B2, B)

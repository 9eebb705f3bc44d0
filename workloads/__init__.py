"""Seeded synthetic inputs for the heterogeneous-adapter LoRA apply.

This module only draws numbers and arranges them: adapter ranks and scales,
dense adapter matrices A (rank x d_in) and B (d_out x rank), activations x,
initial outputs y0, per-token adapter ids and prefill segment layouts.  It holds
none of the method's arithmetic (no products, no sums of products), so that the
fp64 oracle and the HIP path can both consume it without sharing any part of the
computation.

Values are drawn in float64 with numpy's PCG64 and quantised once, with
round-to-nearest-even, to the storage type.  Stored arrays are raw bit patterns
(uint16 for fp16/bf16, float32 for fp32) so that both consumers decode the very
same bytes.

The workloads stand in for the datasets the pages evaluate on (ShareGPT/Alpaca
request streams on LLaMA-7B..70B); they reproduce the shapes, rank mixes,
adapter-popularity laws and request-length mixes, not any dataset's content.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

DTYPES = ("f32", "f16", "bf16", "e4m3")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
# quiet-NaN bit patterns used to poison unused pool memory
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F}


# ----------------------------------------------------------------------------
# quantisation of float64 draws to storage bit patterns (input preparation)
# ----------------------------------------------------------------------------
def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to `dtype` (RNE) and return the stored form."""
    a = np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        f = a.astype(np.float32)  # RNE to fp32 first
        u = f.view(np.uint32).astype(np.uint64)
        r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return r.astype(np.uint16)
    raise ValueError(dtype)


def quantize_e4m3(a: np.ndarray) -> np.ndarray:
    """Round float64 values to OCP FP8 E4M3 codes (uint8), nearest even, with
    magnitudes past the largest finite value (448) saturated to it.  E4M3: sign,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m * 2^-9."""
    a = np.asarray(a, dtype=np.float64)
    sign = np.signbit(a)
    x = np.minimum(np.abs(a), 448.0)
    _, ex = np.frexp(x)                       # x = f * 2^ex, 0.5 <= f < 1
    e = np.clip(ex - 1, -6, 8)                # binade exponent, subnormals share -6
    quantum = np.ldexp(1.0, e - 3)
    r = np.minimum(np.round(x / quantum) * quantum, 448.0)   # np.round: ties to even
    _, rex = np.frexp(r)
    re_ = rex - 1
    normal = (r >= 2.0 ** -6)
    mant = np.where(normal, np.round(np.ldexp(r, -re_) * 8) - 8, np.round(np.ldexp(r, 9)))
    code = np.where(normal, ((re_ + 7) << 3) + mant, mant).astype(np.int64)
    code = np.where(r == 0, 0, code)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def dequantize(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored form -> float64 (exact).  Used by tests and generators only."""
    if dtype == "e4m3":
        b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
        e, m = (b >> 3) & 15, b & 7
        v = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                     np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64)))
        v = np.where((e == 15) & (m == 7), np.nan, v)
        return np.where(b >> 7, -v, v)
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "e4m3": np.uint8}.get(dtype, np.uint16)


# ----------------------------------------------------------------------------
# distributions
# ----------------------------------------------------------------------------
def zipf_ids(rng: np.random.Generator, n: int, n_adapters: int, s: float,
             perm: np.ndarray) -> np.ndarray:
    """Finite Zipf(s) over `n_adapters` items: p(k) ~ k^-s, k = 1..N.
    Popularity rank k maps to adapter id perm[k-1]."""
    k = np.arange(1, n_adapters + 1, dtype=np.float64)
    p = k ** (-s)
    p /= p.sum()
    ranks = rng.choice(n_adapters, size=n, p=p)
    return perm[ranks].astype(np.int32)


def lognormal_lengths(rng: np.random.Generator, count: int, mean: float, total: int,
                      sigma: float = 1.0) -> np.ndarray:
    """`count` request lengths from a lognormal law with the given mean
    (mu = ln(mean) - sigma^2/2), rescaled to sum exactly to `total` with a
    largest-remainder rounding; every length is at least 1."""
    mu = math.log(mean) - 0.5 * sigma * sigma
    raw = rng.lognormal(mu, sigma, size=count)
    share = raw / raw.sum() * (total - count)  # reserve one token per request
    base = np.floor(share).astype(np.int64)
    rem = (total - count) - int(base.sum())
    order = np.argsort(-(share - base), kind="stable")
    base[order[:rem]] += 1
    out = base + 1
    assert int(out.sum()) == total and out.min() >= 1
    return out.astype(np.int32)


def loguniform_ranks(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    r = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n)))
    return np.clip(r, lo, hi).astype(np.int32)


# ----------------------------------------------------------------------------
# workload description
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Batch:
    ids: np.ndarray                     # int32 [n]; -1 = no adapter
    x: List[np.ndarray]                 # per slice, stored bits [n][d_in]
    y0: List[np.ndarray]                # per slice, stored bits [n][d_out] (y dtype)
    seg_lengths: Optional[np.ndarray] = None   # prefill request lengths (token order)
    n_decode: int = 0


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                    # "bgmv" | "sgmv" | "mixed"
    dtype: str                   # weight / activation storage type
    page_elems: int
    slices: List[Tuple[int, int]]   # (d_in, d_out) per slice
    ranks: np.ndarray            # int32 [n_adapters]
    scales: np.ndarray           # float32 [n_adapters]
    seed: int
    shuffle_seed: int
    pool_slack: float            # pool capacity / adapter pages
    kv_dummy_ratio: float        # KV-sized dummy pages per adapter page
    exact: bool = False
    bank: Optional[np.ndarray] = None      # stored-bits weight bank (large configs)
    _bank_offsets: Optional[np.ndarray] = None
    _dense_cache: Dict = dataclasses.field(default_factory=dict)
    act_dtype: Optional[str] = None        # x (and 16-bit y) dtype; default: dtype

    def __post_init__(self):
        if self.act_dtype is None:
            self.act_dtype = self.dtype

    @property
    def quantized(self) -> bool:
        return self.dtype == "e4m3"

    def qscales(self, adapter: int, slice_idx: int):
        """Scales of a quantised adapter slice: (a_scale [r] per rank row of A,
        b_scale [r] per rank column of B), float32; None for other dtypes.
        Drawn per (adapter, slice): 0.02/64 * 2^U(-1/2, 1/2) (codes come from
        N(0, 1) * 64, so the weights are ~N(0, 0.02)); exact mode: powers of
        two in {1/2, 1, 2}."""
        if not self.quantized:
            return None
        r = int(self.ranks[adapter])
        rng = np.random.Generator(np.random.PCG64([self.seed, 7321, slice_idx, adapter]))
        if self.exact:
            sa = 2.0 ** rng.integers(-1, 2, size=r)
            sb = 2.0 ** rng.integers(-1, 2, size=r)
        else:
            sa = 0.02 / 64 * 2.0 ** rng.uniform(-0.5, 0.5, size=r)
            sb = 0.02 / 64 * 2.0 ** rng.uniform(-0.5, 0.5, size=r)
        return sa.astype(np.float32), sb.astype(np.float32)

    @property
    def n_adapters(self) -> int:
        return int(self.ranks.shape[0])

    @property
    def max_rank(self) -> int:
        return int(self.ranks.max())

    def weights(self, adapter: int, slice_idx: int) -> Tuple[np.ndarray, np.ndarray]:
        """Dense stored bits (A [r][d_in], B [d_out][r]) of one adapter slice."""
        key = (adapter, slice_idx)
        if key in self._dense_cache:
            return self._dense_cache[key]
        d_in, d_out = self.slices[slice_idx]
        r = int(self.ranks[adapter])
        na, nb = r * d_in, d_out * r
        if self.bank is not None:
            off = int(self._bank_offsets[slice_idx, adapter])
            flat = self.bank[off: off + na + nb]
            A = flat[:na].reshape(r, d_in)
            B = flat[na:].reshape(d_out, r)
        else:
            rng = np.random.Generator(np.random.PCG64(
                [self.seed, 7919, slice_idx, adapter]))
            if self.exact:
                A = _store(rng.integers(-1, 2, size=(r, d_in)), self.dtype)
                B = _store(rng.integers(-1, 2, size=(d_out, r)), self.dtype)
            elif self.quantized:
                A = quantize_e4m3(rng.normal(0.0, 1.0, size=(r, d_in)) * 64)
                B = quantize_e4m3(rng.normal(0.0, 1.0, size=(d_out, r)) * 64)
            else:
                A = quantize(rng.normal(0.0, 0.02, size=(r, d_in)), self.dtype)
                B = quantize(rng.normal(0.0, 0.02, size=(d_out, r)), self.dtype)
            if len(self._dense_cache) < 64:
                self._dense_cache[key] = (A, B)
        return A, B

    def adapter_pages(self, elt: Optional[int] = None) -> int:
        """Pages all adapters occupy under the pool layout (A rows split into
        ceil(d_in/P) pages; B rows packed floor(P/r_s) per page, r_s = rank
        rounded up to a 16-byte multiple)."""
        elt = ELT_BYTES[self.dtype] if elt is None else elt
        P = self.page_elems
        per16 = 16 // elt
        total = 0
        for d_in, d_out in self.slices:
            npa = -(-d_in // P)
            for r in self.ranks.tolist():
                rs = -(-r // per16) * per16
                rpp = P // rs
                total += r * npa + -(-d_out // rpp)
        return total

    def pool_pages(self) -> int:
        ap = self.adapter_pages()
        return int(math.ceil(ap * (self.pool_slack + self.kv_dummy_ratio)))


# ----------------------------------------------------------------------------
# the five configurations
# ----------------------------------------------------------------------------
CONFIG_NAMES = {
    0: "tiny_bgmv",
    1: "llama7b_decode_bgmv",
    2: "hetero_decode_bgmv",
    3: "llama13b_prefill_sgmv",
    4: "llama70b_mixed_apply",
    # the Llama-7B decode batch with FP8 E4M3 adapter pages (per-row scales)
    5: "llama7b_decode_bgmv_fp8",
}


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored form of float64 draws: RNE to the dtype (E4M3 codes for e4m3)."""
    return quantize_e4m3(a) if dtype == "e4m3" else quantize(a, dtype)


def _ranks_and_scales(cfg: int, rng, exact: bool, alpha: float = 16.0):
    if cfg == 0:
        ranks = np.array([4, 8, 8, 16], np.int32)
    elif cfg in (1, 5):
        ranks = np.full(1000, 16, np.int32)
    elif cfg == 2:
        ranks = rng.choice(np.array([8, 16, 32, 64], np.int32), size=2000)
    elif cfg == 3:
        ranks = rng.choice(np.array([16, 64], np.int32), size=500)
    elif cfg == 4:
        ranks = loguniform_ranks(rng, 2000, 8, 128)
    else:
        raise ValueError(cfg)
    ranks = ranks.astype(np.int32)
    if exact:
        # powers of two keep every product exact in fp32
        scales = np.array([2.0 ** -math.floor(math.log2(r)) for r in ranks], np.float32)
    else:
        scales = (alpha / ranks.astype(np.float64)).astype(np.float32)
    return ranks, scales


def make_workload(cfg: int, exact: bool = False, seed: Optional[int] = None,
                  bank_elems: Optional[int] = None) -> Workload:
    """Build the adapter population of configuration `cfg` (0..4)."""
    seed = 1000 + cfg if seed is None else seed
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    ranks, scales = _ranks_and_scales(cfg, rng, exact)
    if cfg == 0:
        wl = Workload("tiny_bgmv", "bgmv", "f32", 256, [(256, 256)], ranks, scales,
                      seed, shuffle_seed=seed * 31 + 7, pool_slack=2.0,
                      kv_dummy_ratio=0.0, exact=exact)
    elif cfg == 1:
        wl = Workload("llama7b_decode_bgmv", "bgmv", "f16", 4096, [(4096, 4096)] * 4,
                      ranks, scales, seed, shuffle_seed=seed * 31 + 7, pool_slack=1.25,
                      kv_dummy_ratio=0.0, exact=exact)
    elif cfg == 2:
        wl = Workload("hetero_decode_bgmv", "bgmv", "bf16", 4096,
                      [(4096, 4096), (4096, 11008)], ranks, scales, seed,
                      shuffle_seed=seed * 31 + 7, pool_slack=1.05, kv_dummy_ratio=1.0,
                      exact=exact)
    elif cfg == 3:
        wl = Workload("llama13b_prefill_sgmv", "sgmv", "bf16", 5120,
                      [(5120, 5120), (5120, 13824)], ranks, scales, seed,
                      shuffle_seed=seed * 31 + 7, pool_slack=1.25, kv_dummy_ratio=0.0,
                      exact=exact)
    elif cfg == 4:
        wl = Workload("llama70b_mixed_apply", "mixed", "bf16", 8192,
                      [(8192, 8192), (8192, 28672)], ranks, scales, seed,
                      shuffle_seed=seed * 31 + 7, pool_slack=1.05, kv_dummy_ratio=0.0,
                      exact=exact)
    else:
        wl = Workload("llama7b_decode_bgmv_fp8", "bgmv", "e4m3", 4096, [(4096, 4096)] * 4,
                      ranks, scales, seed, shuffle_seed=seed * 31 + 7, pool_slack=1.25,
                      kv_dummy_ratio=0.0, exact=exact, act_dtype="f16")
    # Large populations draw every adapter slice as a window of one iid weight
    # bank at a seeded offset: each window is iid N(0, 0.02) (or {-1,0,1}), and
    # generating thousands of adapters costs one bank instead of one draw each.
    if cfg >= 1:
        need = max(int(r) * (d_in + d_out) for r in ranks for d_in, d_out in wl.slices)
        n_bank = bank_elems or max(1 << 24, 4 * need)
        brng = np.random.Generator(np.random.PCG64([seed, 2]))
        if exact:
            wl.bank = _store(brng.integers(-1, 2, size=n_bank), wl.dtype)
        elif wl.quantized:
            wl.bank = quantize_e4m3(brng.normal(0.0, 1.0, size=n_bank) * 64)
        else:
            wl.bank = quantize(brng.normal(0.0, 0.02, size=n_bank), wl.dtype)
        orng = np.random.Generator(np.random.PCG64([seed, 3]))
        offs = np.zeros((len(wl.slices), wl.n_adapters), np.int64)
        for s, (d_in, d_out) in enumerate(wl.slices):
            sizes = ranks.astype(np.int64) * (d_in + d_out)
            offs[s] = (orng.random(wl.n_adapters) * (n_bank - sizes)).astype(np.int64)
        wl._bank_offsets = offs
    return wl


def _activations(rng, n: int, d: int, dtype: str, exact: bool) -> np.ndarray:
    if exact:
        return quantize(rng.integers(-1, 2, size=(n, d)), dtype)
    return quantize(rng.normal(0.0, 1.0, size=(n, d)), dtype)


def _y0(rng, n: int, d: int, y_dtype: str, exact: bool, zero: bool) -> np.ndarray:
    if zero:
        return quantize(np.zeros((n, d)), y_dtype)
    if exact:
        return quantize(rng.integers(-4, 5, size=(n, d)), y_dtype)
    return quantize(rng.normal(0.0, 1.0, size=(n, d)), y_dtype)


def make_batch(wl: Workload, index: int = 0, y_dtype: Optional[str] = None,
               zero_y0: bool = True, n_tokens: Optional[int] = None,
               slices: Optional[Sequence[int]] = None, with_x: bool = True) -> Batch:
    """Draw batch `index` of the workload: ids (+ segment layout) and, per slice,
    x and y0.  `n_tokens` overrides the token count of BGMV configurations."""
    y_dtype = y_dtype or wl.act_dtype
    rng = np.random.Generator(np.random.PCG64([wl.seed, 100 + index]))
    N = wl.n_adapters
    seg = None
    n_dec = 0
    pop_perm = np.random.Generator(np.random.PCG64([wl.seed, 4])).permutation(N)
    if wl.name == "tiny_bgmv":
        n = n_tokens or 8
        ids = rng.integers(0, N, size=n).astype(np.int32)
    elif wl.name in ("llama7b_decode_bgmv", "llama7b_decode_bgmv_fp8"):
        n = n_tokens or 64
        ids = rng.integers(0, N, size=n).astype(np.int32)
    elif wl.name == "hetero_decode_bgmv":
        n = n_tokens or 256
        ids = zipf_ids(rng, n, N, 1.0, pop_perm)
    elif wl.name == "llama13b_prefill_sgmv":
        total = n_tokens or 8192
        nreq = 32 if total >= 32 else max(1, total // 4)
        lens = lognormal_lengths(rng, nreq, total / nreq, total)
        req_ad = rng.integers(0, N, size=nreq).astype(np.int32)
        # requests sharing an adapter are laid out next to each other
        order = np.argsort(req_ad, kind="stable")
        lens, req_ad = lens[order], req_ad[order]
        ids = np.repeat(req_ad, lens).astype(np.int32)
        seg = lens
        n = int(lens.sum())
    elif wl.name == "llama70b_mixed_apply":
        scale_tokens = (n_tokens or 4608) / 4608.0
        n_pre = max(16, int(round(4096 * scale_tokens)))
        n_dec = max(1, int(round(512 * scale_tokens)))
        lens = lognormal_lengths(rng, 16, n_pre / 16, n_pre)
        seg_ad = zipf_ids(rng, 16, N, 1.2, pop_perm)
        dec_ad = zipf_ids(rng, n_dec, N, 1.2, pop_perm)
        ids = np.concatenate([np.repeat(seg_ad, lens), dec_ad]).astype(np.int32)
        seg = lens
        n = int(ids.shape[0])
    else:
        raise ValueError(wl.name)
    slices = range(len(wl.slices)) if slices is None else slices
    xs, y0s = [], []
    for s in range(len(wl.slices)):
        if s not in slices or not with_x:
            xs.append(None)
            y0s.append(None)
            continue
        d_in, d_out = wl.slices[s]
        srng = np.random.Generator(np.random.PCG64([wl.seed, 200 + index, s]))
        xs.append(_activations(srng, n, d_in, wl.act_dtype, wl.exact))
        y0s.append(_y0(srng, n, d_out, y_dtype, wl.exact, zero_y0))
    return Batch(ids=ids, x=xs, y0=y0s, seg_lengths=seg, n_decode=n_dec)


def small_workload(dtype: str, d_in: int, d_out: int, ranks: Sequence[int], page_elems: int,
                   seed: int = 5, exact: bool = False, alpha: float = 16.0,
                   scales: Optional[Sequence[float]] = None, n_slices: int = 1,
                   pool_slack: float = 2.0, kv_dummy_ratio: float = 0.0,
                   act_dtype: Optional[str] = None) -> Workload:
    """An ad-hoc population for edge-case tests (odd ranks, ragged pages, ...)."""
    ranks = np.asarray(ranks, np.int32)
    if scales is None:
        if exact:
            scales = [2.0 ** -math.floor(math.log2(r)) for r in ranks]
        else:
            scales = [alpha / float(r) for r in ranks]
    if act_dtype is None and dtype == "e4m3":
        act_dtype = "bf16"
    return Workload("custom", "bgmv", dtype, page_elems, [(d_in, d_out)] * n_slices, ranks,
                    np.asarray(scales, np.float32), seed, shuffle_seed=seed * 31 + 7,
                    pool_slack=pool_slack, kv_dummy_ratio=kv_dummy_ratio, exact=exact,
                    act_dtype=act_dtype)


def custom_batch(wl: Workload, ids: Sequence[int], index: int = 0, y_dtype: Optional[str] = None,
                 zero_y0: bool = False) -> Batch:
    y_dtype = y_dtype or wl.act_dtype
    ids = np.asarray(ids, np.int32)
    n = ids.shape[0]
    xs, y0s = [], []
    for s, (d_in, d_out) in enumerate(wl.slices):
        srng = np.random.Generator(np.random.PCG64([wl.seed, 300 + index, s]))
        xs.append(_activations(srng, n, d_in, wl.act_dtype, wl.exact))
        y0s.append(_y0(srng, n, d_out, y_dtype, wl.exact, zero_y0))
    return Batch(ids=ids, x=xs, y0=y0s)

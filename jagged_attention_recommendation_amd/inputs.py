"""Seeded synthetic inputs for jagged attention, shared by the GPU path and the oracle.

This module only draws random numbers and encodes them (bf16 rounding, MX-fp8 quantisation). It
holds none of the attention arithmetic, imports neither the GPU library nor the oracle, and needs
only numpy, so both sides see identical bits.

Workloads follow the shapes the pages describe for a recommendation model's sequence features
(page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model": jagged
user sequences from hundreds to tens of thousands of events; self-, PMA- and cross-attention in
the GDPA paragraph; short or asymmetric K/V in the production-traffic paragraph; MXFP8 in the
low-precision part). The pages hold no length traces, so the distributions below stand in for the
production traffic.

Recipe (per problem): ``rng = numpy.random.default_rng(seed)``; draw the lengths, then Q, K, V, dO
as float32 standard normals in that order (``rng.standard_normal(n, dtype=float32)``), then the bias
table as float32 N(0, 0.02^2). bf16 values are float32 rounded to nearest-even. MX values are
quantised per 32 consecutive elements along the head dimension (OCP MX v1.0): the shared e8m0
exponent is floor(log2(amax)) - 8 (8 = e4m3's largest exponent), elements are rounded to nearest
e4m3 with ties to even and saturated to +-448.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# ----------------------------------------------------------------------------------------------
# length distributions


def lengths_uniform(rng, B, lo, hi):
    """B integer lengths uniform in [lo, hi], both ends inclusive."""
    return rng.integers(lo, hi + 1, size=B).astype(np.int64)


def lengths_lognormal(rng, B, mu, sigma, lo, hi):
    """clip(rint(exp(N(mu, sigma^2))), lo, hi)."""
    x = np.rint(np.exp(rng.normal(mu, sigma, size=B)))
    return np.clip(x, lo, hi).astype(np.int64)


def offsets_from_lengths(lengths):
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    assert off[-1] < 2**31, "offsets must fit int32"
    return off.astype(np.int32)


# ----------------------------------------------------------------------------------------------
# encodings


def bf16_bits(x):
    """float32 array -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits):
    """bf16 bit patterns -> the exact float32 values."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_positive_table():
    """Values of the 127 finite non-negative e4m3 codes 0x00..0x7E, in code order."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = (m / 8.0) * 2.0**-6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()


def e4m3_encode(y):
    """Round values to the nearest e4m3 code (ties to even), saturating to +-448."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first table value >= a
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = (np.signbit(y) & (code != 0)).astype(np.uint8) << np.uint8(7)
    return code | sign


def mx_quantize(x, block=32):
    """x: float array [..., D] -> (e4m3 codes [..., D] uint8, e8m0 scales [..., D/block] uint8).

    Every block is quantised on its own, so large arrays are cut into row chunks that a thread
    pool quantises side by side (numpy releases the interpreter lock inside these operations);
    the bits are those of one pass over the whole array."""
    x = np.asarray(x)
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    if rows >= 1 << 16:
        import concurrent.futures as cf
        flat = x.reshape(rows, x.shape[-1])
        step = 1 << 14
        codes = np.empty(flat.shape, dtype=np.uint8)
        scales = np.empty((rows, x.shape[-1] // block), dtype=np.uint8)

        def run(r0):
            c, s = _mx_quantize(flat[r0:r0 + step], block)
            codes[r0:r0 + step], scales[r0:r0 + step] = c, s

        workers = min(16, os.cpu_count() or 1)
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, range(0, rows, step)))
        return codes.reshape(x.shape), scales.reshape(x.shape[:-1] + (x.shape[-1] // block,))
    return _mx_quantize(x, block)


def _mx_quantize(x, block):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % block == 0
    xb = x.reshape(x.shape[:-1] + (D // block, block))
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8.0
    e = np.where(amax > 0, e, -127.0)
    X = np.clip(e + 127.0, 0, 254).astype(np.int64)
    scale = np.ldexp(1.0, (X - 127))
    codes = e4m3_encode(xb / scale[..., None]).reshape(x.shape)
    return codes, X.astype(np.uint8)


# ----------------------------------------------------------------------------------------------
# problems


@dataclass
class Problem:
    """One jagged attention problem. Tensors are host arrays with [rows, H, D] layout.

    For dtype "bf16" the tensors are bf16 bit patterns (uint16); for "f32" float32; for "mxfp8"
    Q/K/V are e4m3 codes with e8m0 scales in q_scale/k_scale/v_scale ([rows, H, D/32]).
    """
    name: str
    B: int
    H: int
    D: int
    q_off: np.ndarray
    kv_off: np.ndarray
    dtype: str
    act: str
    causal: bool
    scale: float
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    dO: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None  # float32 [H, NB]
    q_scale: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    seeds: Optional[np.ndarray] = None  # shared query block [max_q, H, D] (PMA), or None
    meta: dict = field(default_factory=dict)

    @property
    def total_q(self):
        return int(self.q_off[-1])

    @property
    def total_kv(self):
        return int(self.kv_off[-1])

    @property
    def lq(self):
        return np.diff(self.q_off.astype(np.int64))

    @property
    def lk(self):
        return np.diff(self.kv_off.astype(np.int64))


def _normal(rng, shape):
    return rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)


def make_problem(name, *, seed, H, D, lq, lk, dtype="bf16", act="softmax", causal=False,
                 bias_buckets=0, with_grad=True, shared_q=False, scale=None):
    """Draw one problem. lq/lk: per-sample lengths, or a callable rng -> lengths.

    shared_q: one block of max(Lq) seed rows is every sample's query block (PMA seeds): local
    query i of each sample is seed row i. p.seeds holds the block; p.Q holds it materialised per
    sample (the jagged layout), so both the shared and the per-sample call can be made.
    """
    rng = np.random.default_rng(seed)
    lq = np.asarray(lq(rng) if callable(lq) else lq, dtype=np.int64)
    lk = np.asarray(lk(rng) if callable(lk) else lk, dtype=np.int64)
    assert lq.shape == lk.shape
    B = len(lq)
    q_off, kv_off = offsets_from_lengths(lq), offsets_from_lengths(lk)
    tq, tk = int(q_off[-1]), int(kv_off[-1])
    seeds = None
    if shared_q:
        seeds = _normal(rng, (max(int(lq.max()) if B > 0 else 1, 1), H, D))
        local = np.concatenate([np.arange(n) for n in lq]) if B > 0 else np.zeros(0, np.int64)
        Qf = seeds[local]
    else:
        Qf = _normal(rng, (tq, H, D))
    Kf = _normal(rng, (tk, H, D))
    Vf = _normal(rng, (tk, H, D))
    dOf = _normal(rng, (tq, H, D)) if with_grad else None
    bias = None
    if bias_buckets > 0:
        bias = (0.02 * _normal(rng, (H, bias_buckets))).astype(np.float32)
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    p = Problem(name=name, B=B, H=H, D=D, q_off=q_off, kv_off=kv_off, dtype=dtype, act=act,
                causal=causal, scale=scale, Q=None, K=None, V=None, bias=bias)
    if seeds is not None:
        p.seeds = bf16_bits(seeds) if dtype == "bf16" else seeds
    if dtype == "f32":
        p.Q, p.K, p.V = Qf, Kf, Vf
        p.dO = dOf
    elif dtype == "bf16":
        p.Q, p.K, p.V = bf16_bits(Qf), bf16_bits(Kf), bf16_bits(Vf)
        p.dO = bf16_bits(dOf) if dOf is not None else None
    elif dtype == "mxfp8":
        p.Q, p.q_scale = mx_quantize(Qf)
        p.K, p.k_scale = mx_quantize(Kf)
        p.V, p.v_scale = mx_quantize(Vf)
        p.dO = bf16_bits(dOf) if dOf is not None else None
    else:
        raise ValueError(dtype)
    return p


# The five workloads. Scale is 1/sqrt(D) throughout; causal only where stated.
CONFIG_NAMES = {
    1: "tiny GDPA self-attention fp32 (B=4 H=2 D=32 L~U[1,64] SiLU)",
    2: "JFA softmax causal self-attention bf16 (B=64 H=4 D=128 L~U[1,2048] bias[4,4096])",
    3: "GDPA cross-attention bf16 (B=256 H=4 D=128 Lq~U[64,4096] Lk~U[8,64] GELU-tanh)",
    4: "PMA GDPA bf16 (B=512 H=8 D=64 Lq=32 shared seeds Lk~lognormal(6,1.2) in [16,16384] SiLU)",
    5: "MX-fp8 causal self-attention fwd (B=128 H=8 D=128 L~lognormal(7,1.0) in [16,16384])",
}


def config_problem(k, act=None, B=None, seed=None, with_grad=None):
    """Problem for workload k (1..5). B overrides the sample count (same per-sample recipe).
    with_grad=True also draws dO for the forward-only workloads (1 and 5); it is drawn after V and
    before any bias, so Q, K and V keep their bits."""
    seed = 1000 + k if seed is None else seed
    if k == 1:
        b = 4 if B is None else B
        u = lambda rng: lengths_uniform(rng, b, 1, 64)
        return _same_len_problem("config1", seed, b, 2, 32, u, dtype="f32", act=act or "silu",
                                 causal=False, bias_buckets=0, with_grad=bool(with_grad))
    if k == 2:
        b = 64 if B is None else B
        u = lambda rng: lengths_uniform(rng, b, 1, 2048)
        return _same_len_problem("config2", seed, b, 4, 128, u, dtype="bf16",
                                 act=act or "softmax", causal=True, bias_buckets=4096)
    if k == 3:
        b = 256 if B is None else B

        def both(rng):
            return lengths_uniform(rng, b, 64, 4096), lengths_uniform(rng, b, 8, 64)
        return _pair_len_problem("config3", seed, b, 4, 128, both, act=act or "gelu_tanh")
    if k == 4:
        b = 512 if B is None else B

        def both(rng):
            return np.full(b, 32, np.int64), lengths_lognormal(rng, b, 6.0, 1.2, 16, 16384)
        return _pair_len_problem("config4", seed, b, 8, 64, both, act=act or "silu", shared_q=True)
    if k == 5:
        b = 128 if B is None else B
        u = lambda rng: lengths_lognormal(rng, b, 7.0, 1.0, 16, 16384)
        return _same_len_problem("config5", seed, b, 8, 128, u, dtype="mxfp8",
                                 act=act or "softmax", causal=True, bias_buckets=0,
                                 with_grad=bool(with_grad))
    raise ValueError(k)


def _same_len_problem(name, seed, B, H, D, draw, **kw):
    cache = {}

    def lq(rng):
        cache["l"] = draw(rng)
        return cache["l"]

    def lk(rng):
        return cache["l"]
    return make_problem(name, seed=seed, H=H, D=D, lq=lq, lk=lk, **kw)


def _pair_len_problem(name, seed, B, H, D, draw_both, **kw):
    cache = {}

    def lq(rng):
        cache["q"], cache["k"] = draw_both(rng)
        return cache["q"]

    def lk(rng):
        return cache["k"]
    return make_problem(name, seed=seed, H=H, D=D, lq=lq, lk=lk, dtype="bf16", **kw)


def as_f64(p: Problem, which: str):
    """Exact fp64 view of a problem tensor for the oracle (bf16/f32 upcast; MX left encoded)."""
    a = getattr(p, which)
    if a is None:
        return None
    if p.dtype == "bf16" or (p.dtype == "mxfp8" and which == "dO"):
        return bf16_to_f32(a).astype(np.float64)
    if p.dtype == "f32":
        return a.astype(np.float64)
    raise ValueError("MX tensors are decoded by the consumer")

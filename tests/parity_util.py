"""Helpers for GPU-vs-oracle parity tests (test infrastructure).

Tolerance: an element g of a GPU output and the oracle's r agree when
|g - r| <= atol * s + rtol * |r|, where s = max(1, rms of r over the output's (sample, head)
block). The rms term keeps the check meaningful for GDPA, whose outputs are unnormalised sums of
up to thousands of terms; for softmax outputs s is 1. bf16 results use atol = rtol = 2e-2 (half a
bf16 ulp is 2^-9 ~ 2e-3 per rounding, and P is rounded to bf16 before the second product), fp32
results 1e-4 / 1e-4, lse 1e-3 / 1e-4. These numbers were fixed before any kernel ran.

One reading was added later, after a GPU result failed: the rms is taken over the block's rows
that form a sum, i.e. rows with at least one valid (query, key) pair. A row that forms no sum (a
key that no query reaches under a causal mask when Lq < Lk, a query with no valid key) carries no
rounding, and counting it diluted s for the rows that do. A dV element of a causal SiLU sample
with 40 queries and 350 keys exceeded the diluted bound by 13 %; tests/test_tolerance.py rounds P
to bf16 on the CPU for such a sample and shows that this rounding alone produces errors of that
size, and that the rows forming no sum stay exactly zero. Because the wider s would otherwise
also admit stray values on those rows, the parity checks pass the rows that form a sum
(live_q_rows / live_k_rows) and every other row must be exactly zero on the GPU. A row that forms
a sum can still be exactly zero in the oracle by cancellation (the softmax gradient of a query
with a single valid key); it keeps the ordinary bound.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from jagged_attention_recommendation_amd import inputs

TOL = {
    "f32": (1e-4, 1e-4),
    "bf16": (2e-2, 2e-2),
    "mxfp8": (2e-2, 2e-2),
    "lse": (1e-3, 1e-4),
}


def to_device(p, device="cuda"):
    """Upload a Problem's host arrays (identical bits) to the GPU."""
    def t(a, kind):
        if a is None:
            return None
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        if kind == "u8":
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    kind = {"bf16": "bf16", "f32": "f32", "mxfp8": "u8"}[p.dtype]
    d = {
        "Q": t(p.Q, kind), "K": t(p.K, kind), "V": t(p.V, kind),
        "dO": t(p.dO, "bf16" if p.dtype != "f32" else "f32"),
        "q_off": torch.from_numpy(p.q_off.astype(np.int32)).to(device),
        "kv_off": torch.from_numpy(p.kv_off.astype(np.int32)).to(device),
        "bias": torch.from_numpy(p.bias).to(device) if p.bias is not None else None,
        "q_scale": t(p.q_scale, "u8"), "k_scale": t(p.k_scale, "u8"), "v_scale": t(p.v_scale, "u8"),
    }
    return d


def host_f64(p, which):
    """Exact fp64 values of a problem tensor (MX decoded by the oracle's own decoder)."""
    if p.dtype == "mxfp8" and which in ("Q", "K", "V"):
        return oracle.decode_mx(getattr(p, which), getattr(p, which[0].lower() + "_scale"))
    return inputs.as_f64(p, which)


def oracle_fwd(p, nthreads=None):
    return oracle.fwd(p.q_off, p.kv_off, host_f64(p, "Q"), host_f64(p, "K"), host_f64(p, "V"),
                      act=p.act, causal=p.causal, scale=p.scale,
                      bias=None if p.bias is None else p.bias.astype(np.float64), nthreads=nthreads)


def oracle_bwd(p, nthreads=None):
    return oracle.bwd(p.q_off, p.kv_off, host_f64(p, "Q"), host_f64(p, "K"), host_f64(p, "V"),
                      host_f64(p, "dO"), act=p.act, causal=p.causal, scale=p.scale,
                      bias=None if p.bias is None else p.bias.astype(np.float64), nthreads=nthreads,
                      error_scale=True)


def block_scale(r, off, live=None):
    """s[row, h] = max(1, rms of r over the rows of the (sample, head) block containing that row
    that form a sum: the `live` rows when given, else the rows whose value is nonzero)."""
    rows, H = r.shape[0], r.shape[1]
    s = np.ones((rows, H))
    for b in range(len(off) - 1):
        lo, hi = int(off[b]), int(off[b + 1])
        if hi > lo:
            blk = r[lo:hi].reshape(hi - lo, H, -1)
            sq = (blk ** 2).sum(axis=2)                  # [rows, H]
            if live is not None:
                active = np.full(H, int(np.count_nonzero(live[lo:hi])))
            else:
                active = (blk != 0).any(axis=2).sum(axis=0)  # rows forming a sum, per head
            rms = np.sqrt(sq.sum(axis=0) / np.maximum(active * blk.shape[2], 1))
            s[lo:hi] = np.maximum(1.0, rms)[None, :]
    return s


def live_q_rows(q_off, kv_off, causal, window=0):
    """Query rows that form a sum: at least one valid key. With a causal mask key 0 is valid for
    every query when the sample has a key; a window of W keys (W below the query count) also
    drops queries i >= Lk - 1 + W, whose window lies past the last key."""
    out = np.zeros(int(q_off[-1]), dtype=bool)
    for b in range(len(q_off) - 1):
        lo, hi = int(q_off[b]), int(q_off[b + 1])
        Lk = int(kv_off[b + 1] - kv_off[b])
        if Lk == 0:
            continue
        i = np.arange(hi - lo)
        ok = np.ones(hi - lo, dtype=bool)
        if causal and window > 0:
            ok = i < Lk - 1 + window
        out[lo:hi] = ok
    return out


def live_k_rows(q_off, kv_off, causal, window=0):
    """Key rows that form a sum: reached by at least one query (causal: j < Lq; the query j
    itself is always inside j's window)."""
    out = np.zeros(int(kv_off[-1]), dtype=bool)
    for b in range(len(q_off) - 1):
        lo, hi = int(kv_off[b]), int(kv_off[b + 1])
        Lq = int(q_off[b + 1] - q_off[b])
        if Lq == 0:
            continue
        j = np.arange(hi - lo)
        out[lo:hi] = j < Lq if causal else True
    return out


def live_rows(p, side, window=0):
    f = live_q_rows if side == "q" else live_k_rows
    return f(p.q_off, p.kv_off, p.causal, window)


def assert_close(g, r, off, kind, name, live=None):
    """Element-wise tolerance check; g may be a torch tensor (any float dtype). live: rows that
    form a sum (bool per row); every other row must be exactly zero, and the block rms is taken
    over the live rows. Without it the rms is taken over the rows whose oracle value is
    nonzero."""
    if isinstance(g, torch.Tensor):
        g = g.detach().float().cpu().numpy().astype(np.float64)
    atol, rtol = TOL[kind]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    if g.ndim == 3:
        s = block_scale(r, off, live)[..., None]
    else:
        s = np.ones_like(r)
    err = np.abs(g - r)
    bound = atol * s + rtol * np.abs(r)
    if live is not None:
        live = np.asarray(live, dtype=bool)
        assert live.shape == (r.shape[0],)
        assert not r[~live].any(), f"{name}: the oracle has values on rows that form no sum"
        bound[~live] = 0.0
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} elements out of tolerance; "
                             f"max abs err {err.max():.3e}; first bad {idx.tolist()} "
                             f"g={g[tuple(idx[0])]:.6g} r={r[tuple(idx[0])]:.6g}")
    return float(err.max())


def assert_lse_close(g, r, name="lse"):
    if isinstance(g, torch.Tensor):
        g = g.detach().double().cpu().numpy()
    atol, rtol = TOL["lse"]
    neg = np.isneginf(r)
    assert np.array_equal(np.isneginf(g), neg), f"{name}: -inf pattern differs"
    err = np.abs(g[~neg] - r[~neg])
    bound = atol + rtol * np.abs(r[~neg])
    assert (err <= bound).all(), f"{name}: max err {err.max():.3e}"


def subproblem(p, b, heads=None):
    """Sample b of p as a one-sample problem (same bits), optionally restricted to some heads."""
    import copy
    q = slice(int(p.q_off[b]), int(p.q_off[b + 1]))
    k = slice(int(p.kv_off[b]), int(p.kv_off[b + 1]))
    hs = slice(None) if heads is None else heads
    sp = copy.copy(p)
    sp.B = 1
    sp.q_off = np.array([0, q.stop - q.start], np.int32)
    sp.kv_off = np.array([0, k.stop - k.start], np.int32)
    for name, sl in (("Q", q), ("K", k), ("V", k), ("dO", q), ("q_scale", q), ("k_scale", k),
                     ("v_scale", k)):
        a = getattr(p, name)
        if a is not None:
            setattr(sp, name, np.ascontiguousarray(a[sl][:, hs]))
    if p.bias is not None:
        sp.bias = np.ascontiguousarray(p.bias[hs])
    sp.H = sp.Q.shape[1]
    return sp

"""Work and traffic counters for jagged attention problems (used for reporting, not compute).

"Useful" work counts only the matrix-product flops of unmasked (query, key) pairs, the way the
pages measure kernels in isolation on one GPU (page "GEM Training: How Meta Doubled the Efficiency
of Its LLM-Scale Ads Foundation Model", local-MFU part): forward = 2 products = 4*D flops per pair
and head; backward = 5 products = 10*D flops per pair and head. Padding, recomputation and
transcendentals are not counted.
"""
from __future__ import annotations

import numpy as np


def pairs_per_sample(lq, lk, causal, window=0):
    """Unmasked (i, j) pairs per sample. Causal keeps j <= i on local positions; a sliding window
    W >= 1 (with causal) also drops keys j <= i - W."""
    lq = np.asarray(lq, dtype=np.int64)
    lk = np.asarray(lk, dtype=np.int64)
    if not causal:
        return lq * lk
    m = np.minimum(lq, lk)
    if window <= 0:
        # sum_{i < Lq} min(i + 1, Lk)
        full = m * (m + 1) // 2                 # rows i < m see i + 1 keys
        rest = np.maximum(lq - lk, 0) * lk      # rows i >= Lk see all Lk keys
        return full + rest
    W = int(window)
    # rows i < m see min(i + 1, W) keys
    head = np.where(m <= W, m * (m + 1) // 2, W * (W + 1) // 2 + (m - W) * W)
    # rows i = Lk + t (t < Lq - Lk) see keys max(0, i - W + 1) .. Lk - 1: min(Lk, max(0, W - 1 - t))
    # of them, i.e. g(W - 1) - g(W - 1 - Lk) with g(a) = sum_t max(0, a - t)
    n = np.maximum(lq - lk, 0)

    def g(a):
        a = np.maximum(a, 0)
        return np.where(n >= a, a * (a + 1) // 2, n * a - n * (n - 1) // 2)
    return head + g(W - 1 + 0 * lk) - g(W - 1 - lk)


def useful_flops(p, direction="fwd", window=0):
    pairs = int(pairs_per_sample(p.lq, p.lk, p.causal, window).sum())
    per = {"fwd": 4, "bwd": 10, "fwdbwd": 14}[direction]
    return float(per) * p.D * p.H * pairs


def elem_bytes(p):
    return {"f32": 4, "bf16": 2, "mxfp8": 1}[p.dtype]


def q_read_rows(p):
    """Rows of Q a pass reads: the shared seed block when the problem has one, else every query."""
    return p.seeds.shape[0] if getattr(p, "seeds", None) is not None else p.total_q


def fwd_bytes(p):
    """Each input read once and each output written once (the algorithmic minimum)."""
    e_in = elem_bytes(p)
    e_out = 4 if p.dtype == "f32" else 2
    H, D = p.H, p.D
    b = (q_read_rows(p) * H * D * e_in + 2 * p.total_kv * H * D * e_in
         + p.total_q * H * D * e_out)
    if p.dtype == "mxfp8":
        b += (p.total_q + 2 * p.total_kv) * H * (D // 32)
    if p.act == "softmax":
        b += p.total_q * H * 4  # lse
    if p.bias is not None:
        b += p.bias.size * 4
    return float(b)


def bwd_bytes(p):
    """Reads Q, K, V, dO (+ O, lse, and D written then read, for softmax); writes dQ, dK, dV.
    With a shared seed block, Q and dQ are that block."""
    e = elem_bytes(p)
    H, D = p.H, p.D
    tq, tk, rq = p.total_q, p.total_kv, q_read_rows(p)
    b = ((rq + tq) * H * D * e + 2 * tk * H * D * e   # Q, dO, K, V
         + rq * H * D * e + 2 * tk * H * D * e)       # dQ, dK, dV
    if p.act == "softmax":
        b += tq * H * D * e + tq * H * 4 + 2 * tq * H * 4  # O, lse, D write + read
    if p.bias is not None:
        b += 2 * p.bias.size * 4
    return float(b)


def kernel_bytes(p, kernel):
    """Algorithmic HBM bytes of one launch of a kernel: every operand it must read and every
    result it must write, each once.

    fwd: Q, K, V read, O (+ lse) written. dq: Q, dO, K, V (+ O and lse for softmax, whose
    prologue forms D) read, dQ (+ D) written. dkdv: Q, dO, K, V (+ lse, D) read, dK, dV written.
    With a shared seed block Q is that block, and the dq kernel's result is every sample's query
    gradient in fp32 (summed over samples by a small reduction afterwards).
    """
    if kernel == "fwd":
        return fwd_bytes(p)
    e = elem_bytes(p)
    H, D = p.H, p.D
    tq, tk, rq = p.total_q, p.total_kv, q_read_rows(p)
    b = (rq + tq + 2 * tk) * H * D * e
    sm = p.act == "softmax"
    if kernel == "dq":
        b += tq * H * D * (4 if getattr(p, "seeds", None) is not None else e)
        if sm:
            b += tq * H * D * e + tq * H * 4 + tq * H * 4
    elif kernel == "dkdv":
        b += 2 * tk * H * D * e
        if sm:
            b += 2 * tq * H * 4
    else:
        raise ValueError(kernel)
    return float(b)


def block_lengths(lengths, block=64):
    """Lengths of the fixed blocks every sample is cut into (the last one of a sample shorter)."""
    out = []
    for L in np.asarray(lengths, dtype=np.int64):
        out.extend([block] * int(L // block))
        if L % block:
            out.append(int(L % block))
    return np.asarray(out, dtype=np.int64)


def block_flops(p, direction="fwd", block=64):
    """Useful flops of block-aligned attention over p's samples: pairs inside each block (causal
    when p is), 4*D per pair and head forward, 10*D backward."""
    bl = block_lengths(p.lq, block)
    pairs = int(pairs_per_sample(bl, bl, p.causal).sum())
    return float({"fwd": 4, "bwd": 10}[direction]) * p.D * p.H * pairs


def block_bytes(p, direction="fwd"):
    """Algorithmic HBM bytes of block-aligned attention (bf16): forward reads Q, K, V and writes
    O; backward reads Q, K, V, dO and writes dQ, dK, dV. No lse or row term touches HBM."""
    per = p.total_q * p.H * p.D * 2
    return float(per * (4 if direction == "fwd" else 7))

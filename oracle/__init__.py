"""Reference oracle for jagged attention: plain fp64 CPU loops, written from the method's definition.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this package. The GPU library never does, and the two share no code.

The C source (``gdpa_oracle.c``) holds the definition and its citations: JFA is FlashAttention on
jagged tensors (page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation
Model", JFA paragraph), so its result is the plain softmax attention over each sample's valid keys;
GDPA (same page, GDPA paragraph) replaces softmax by an element-wise GELU or SiLU with no
normalisation. This module only marshals numpy arrays into that library.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdpa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ACT_SOFTMAX, ACT_GELU_TANH, ACT_SILU = 0, 1, 2
ACTS = {"softmax": ACT_SOFTMAX, "gelu_tanh": ACT_GELU_TANH, "silu": ACT_SILU}

_lib = None


def build(src=None, out=None) -> str:
    """Compile the oracle with gcc (plain C, -O2, OpenMP). Always recompiles. `src` and `out`
    default to this package's source and library; the planted-mistake tests compile altered
    copies of the source elsewhere."""
    src = src or _SRC
    out = out or _LIB_PATH
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(path):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    up = ctypes.POINTER(ctypes.c_uint8)
    c_int, c_long, c_double = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.gdpa_oracle_fwd.argtypes = [c_int, c_int, c_int, ip, ip, dp, dp, dp, dp, c_int, c_int,
                                    c_int, c_int, c_double, dp, dp, c_int]
    lib.gdpa_oracle_fwd.restype = c_int
    lib.gdpa_oracle_bwd.argtypes = [c_int, c_int, c_int, ip, ip, dp, dp, dp, dp, dp, c_int, c_int,
                                    c_int, c_int, c_double, dp, dp, dp, dp, dp, dp, c_int]
    lib.gdpa_oracle_bwd.restype = c_int
    lib.gdpa_oracle_act.argtypes = [c_int, dp, c_long, dp, dp]
    lib.gdpa_oracle_act.restype = None
    lib.gdpa_oracle_decode_e4m3.argtypes = [up, c_long, dp]
    lib.gdpa_oracle_decode_e4m3.restype = None
    lib.gdpa_oracle_decode_e8m0.argtypes = [up, c_long, dp]
    lib.gdpa_oracle_decode_e8m0.restype = None
    lib.gdpa_oracle_decode_mx.argtypes = [up, up, c_long, c_int, dp]
    lib.gdpa_oracle_decode_mx.restype = c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    _lib = _bind(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Run the oracle's functions on another build of its source (the planted-mistake tests load
    a copy with one deliberate error and check that the pins reject it)."""
    global _lib
    saved = _lib
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _act_code(act):
    return ACTS[act] if isinstance(act, str) else int(act)


def fwd(q_off, kv_off, Q, K, V, *, act="softmax", causal=False, scale=None, bias=None,
        nthreads=None, window=0):
    """Forward pass. Q: [total_q, H, D], K/V: [total_kv, H, D] (any float dtype, upcast exactly).
    window W >= 1 also drops keys j <= i - W (sliding window).

    Returns (O [total_q, H, D] fp64, lse [total_q, H] fp64; lse is 0 for GDPA).
    """
    lib = _load()
    q_off, kv_off = _i32(q_off), _i32(kv_off)
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B = len(q_off) - 1
    assert len(kv_off) == B + 1
    total_q, H, D = Q.shape
    assert K.shape == V.shape and K.shape[1:] == (H, D)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    nb = 0
    bias_arr = np.zeros(1)
    if bias is not None:
        bias_arr = _f64(bias)
        assert bias_arr.shape[0] == H
        nb = bias_arr.shape[1]
    O = np.empty((total_q, H, D), dtype=np.float64)
    lse = np.empty((total_q, H), dtype=np.float64)
    rc = lib.gdpa_oracle_fwd(B, H, D, _ptr(q_off, ctypes.c_int32), _ptr(kv_off, ctypes.c_int32),
                             _ptr(Q, ctypes.c_double), _ptr(K, ctypes.c_double),
                             _ptr(V, ctypes.c_double), _ptr(bias_arr, ctypes.c_double), nb,
                             _act_code(act), int(bool(causal)), int(window), float(scale),
                             _ptr(O, ctypes.c_double), _ptr(lse, ctypes.c_double),
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle fwd rejected its arguments (rc={rc})")
    return O, lse


def bwd(q_off, kv_off, Q, K, V, dO, *, act="softmax", causal=False, scale=None, bias=None,
        nthreads=None, error_scale=False, window=0):
    """Backward pass of the loss sum(dO * O).

    Returns dict with dQ, dK, dV (fp64, same layouts as Q/K/V), dbias ([H, NB] or None),
    dbias_scale ([H, NB] or None: the error scale of each bias bucket under a rounded forward
    output, see the C source; computed when error_scale) and D ([total_q, H], the softmax row term sum_j p_ij dp_ij; 0 for
    GDPA).
    """
    lib = _load()
    q_off, kv_off = _i32(q_off), _i32(kv_off)
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B = len(q_off) - 1
    total_q, H, D = Q.shape
    total_kv = K.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    nb = 0
    bias_arr = np.zeros(1)
    dbias = np.zeros(1)
    dscale = np.zeros(1)
    if bias is not None:
        bias_arr = _f64(bias)
        nb = bias_arr.shape[1]
        dbias = np.empty((H, nb), dtype=np.float64)
        dscale = np.empty((H, nb), dtype=np.float64)
    dQ = np.empty((total_q, H, D))
    dK = np.empty((total_kv, H, D))
    dV = np.empty((total_kv, H, D))
    Dv = np.empty((total_q, H))
    rc = lib.gdpa_oracle_bwd(B, H, D, _ptr(q_off, ctypes.c_int32), _ptr(kv_off, ctypes.c_int32),
                             _ptr(Q, ctypes.c_double), _ptr(K, ctypes.c_double),
                             _ptr(V, ctypes.c_double), _ptr(dO, ctypes.c_double),
                             _ptr(bias_arr, ctypes.c_double), nb, _act_code(act),
                             int(bool(causal)), int(window), float(scale), _ptr(dQ, ctypes.c_double),
                             _ptr(dK, ctypes.c_double), _ptr(dV, ctypes.c_double),
                             _ptr(dbias, ctypes.c_double), _ptr(Dv, ctypes.c_double),
                             _ptr(dscale, ctypes.c_double) if error_scale and nb > 0 else None,
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle bwd rejected its arguments (rc={rc})")
    return {"dQ": dQ, "dK": dK, "dV": dV, "dbias": dbias if nb > 0 else None,
            "dbias_scale": dscale if error_scale and nb > 0 else None, "D": Dv}


def shared_rows(q_off, seeds):
    """Per-sample query rows of a shared query block: local query i of every sample is row i of
    `seeds` [max_q, H, D] (PMA: one set of learned seed queries attends to each sample's keys;
    page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model",
    GDPA paragraph). Returns the jagged [total_q, H, D] block."""
    q_off = np.asarray(q_off, dtype=np.int64)
    lens = np.diff(q_off)
    assert (lens <= seeds.shape[0]).all(), "a sample is longer than the shared block"
    idx = np.concatenate([np.arange(n) for n in lens]) if len(lens) else np.zeros(0, np.int64)
    return np.asarray(seeds)[idx]


def fwd_shared_q(q_off, kv_off, seeds, K, V, **kw):
    """Forward with a shared query block (see shared_rows): the plain forward of the expanded
    queries."""
    return fwd(q_off, kv_off, shared_rows(q_off, seeds), K, V, **kw)


def bwd_shared_q(q_off, kv_off, seeds, K, V, dO, **kw):
    """Backward with a shared query block. The loss reaches seed row i through every sample that
    reads it, so its gradient is the sum over those samples of their query gradients (chain rule);
    summed here sample by sample in fp64. Other outputs as in bwd(); dQ is [max_q, H, D]."""
    g = bwd(q_off, kv_off, shared_rows(q_off, seeds), K, V, dO, **kw)
    dq = np.zeros(np.shape(seeds), dtype=np.float64)
    q_off = np.asarray(q_off, dtype=np.int64)
    for b in range(len(q_off) - 1):
        lo, hi = int(q_off[b]), int(q_off[b + 1])
        dq[:hi - lo] += g["dQ"][lo:hi]
    g["dQ"] = dq
    return g


def rope_angles(pos, D, base=10000.0):
    """Rotary position embedding angles [rows, D/2]: pair m of a row at position p turns by
    p * base**(-2m/D). The pages name the rotary embedding but give no formula; this is the
    rotary form of Su et al. (RoFormer), with consecutive elements (2m, 2m+1) as the pairs."""
    assert D % 2 == 0
    m = np.arange(D // 2, dtype=np.float64)
    inv = base ** (-2.0 * m / D)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, pos, base=10000.0):
    """Rotate each (2m, 2m+1) pair of x [rows, H, D] by its row's angle (see rope_angles)."""
    x = _f64(x)
    th = rope_angles(pos, x.shape[2], base)[:, None, :]
    c, s = np.cos(th), np.sin(th)
    e, o = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = c * e - s * o
    y[..., 1::2] = s * e + c * o
    return y


def rope_bwd(g, pos, base=10000.0):
    """Gradient through rope(): each pair's rotation is orthogonal, so the gradient with respect
    to the input is the gradient rotated back (the transpose, i.e. the angle negated)."""
    g = _f64(g)
    th = rope_angles(pos, g.shape[2], base)[:, None, :]
    c, s = np.cos(th), np.sin(th)
    e, o = g[..., 0::2], g[..., 1::2]
    y = np.empty_like(g)
    y[..., 0::2] = c * e + s * o
    y[..., 1::2] = -s * e + c * o
    return y


def local_positions(off):
    """Position of every row inside its sample."""
    off = np.asarray(off, dtype=np.int64)
    lens = np.diff(off)
    return np.concatenate([np.arange(n) for n in lens]) if len(lens) else np.zeros(0, np.int64)


def block_offsets(off, block=64):
    """Offsets of the fixed-size blocks of every sample: sample b's rows are cut into blocks of
    `block` consecutive tokens (the last one shorter). In block-aligned attention (page "GEM
    Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model", block-
    attention paragraph) a query block attends only to the key block at the same place, so the
    blocks are independent attention problems."""
    off = np.asarray(off, dtype=np.int64)
    out = [0]
    for b in range(len(off) - 1):
        L = int(off[b + 1] - off[b])
        for s0 in range(0, L, block):
            out.append(out[-1] + min(block, L - s0))
    return np.asarray(out, dtype=np.int64)


def block_fwd(off, Q, K, V, *, act="softmax", causal=False, scale=None, block=64, rotary=True,
              base=10000.0, nthreads=None):
    """Block-aligned self-attention with rotary embeddings: Q and K are rotated at their
    positions in the sample, then every block of `block` tokens attends within itself (causal:
    also j <= i). Q, K, V: [total, H, D] over the sample offsets `off`. Returns (O, lse)."""
    pos = local_positions(off)
    Qr = rope(Q, pos, base) if rotary else _f64(Q)
    Kr = rope(K, pos, base) if rotary else _f64(K)
    bo = block_offsets(off, block)
    return fwd(bo, bo, Qr, Kr, V, act=act, causal=causal, scale=scale, nthreads=nthreads)


def block_bwd(off, Q, K, V, dO, *, act="softmax", causal=False, scale=None, block=64,
              rotary=True, base=10000.0, nthreads=None):
    """Backward of sum(dO * O) for block_fwd: the blocks' gradients with respect to the rotated
    Q and K, rotated back (rope_bwd). Returns dict with dQ, dK, dV."""
    pos = local_positions(off)
    Qr = rope(Q, pos, base) if rotary else _f64(Q)
    Kr = rope(K, pos, base) if rotary else _f64(K)
    bo = block_offsets(off, block)
    g = bwd(bo, bo, Qr, Kr, V, dO, act=act, causal=causal, scale=scale, nthreads=nthreads)
    dQ = rope_bwd(g["dQ"], pos, base) if rotary else g["dQ"]
    dK = rope_bwd(g["dK"], pos, base) if rotary else g["dK"]
    return {"dQ": dQ, "dK": dK, "dV": g["dV"]}


def act(name, x, derivative=False):
    """The oracle's own activation (or its derivative) on an array."""
    lib = _load()
    x = _f64(x)
    out = np.empty_like(x)
    if derivative:
        lib.gdpa_oracle_act(_act_code(name), _ptr(x, ctypes.c_double), x.size, None,
                            _ptr(out, ctypes.c_double))
    else:
        lib.gdpa_oracle_act(_act_code(name), _ptr(x, ctypes.c_double), x.size,
                            _ptr(out, ctypes.c_double), None)
    return out


def decode_e4m3(codes):
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    lib.gdpa_oracle_decode_e4m3(_ptr(codes, ctypes.c_uint8), codes.size, _ptr(out, ctypes.c_double))
    return out


def decode_e8m0(codes):
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    lib.gdpa_oracle_decode_e8m0(_ptr(codes, ctypes.c_uint8), codes.size, _ptr(out, ctypes.c_double))
    return out


def decode_mx(data, scales):
    """data: [..., D] e4m3 codes, scales: [..., D/32] e8m0 codes -> fp64 values [..., D]."""
    lib = _load()
    data = np.ascontiguousarray(data, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    D = data.shape[-1]
    rows = data.size // D
    assert scales.shape[-1] * 32 == D and scales.size // scales.shape[-1] == rows
    out = np.empty(data.shape, dtype=np.float64)
    rc = lib.gdpa_oracle_decode_mx(_ptr(data, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), rows,
                                   D, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle decode_mx: D must be a multiple of 32")
    return out

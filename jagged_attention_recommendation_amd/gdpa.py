"""Thin ctypes binding of libgdpa.so (C ABI in include/gdpa.h).

Argument marshalling only: every step of forward and backward runs in the library's HIP kernels.
torch provides device memory and the current stream. There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported first so libgdpa.so binds to the HIP runtime torch has loaded

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdpa.so")

ACT = {"softmax": 0, "gelu_tanh": 1, "silu": 2}
DTYPE = {"f32": 0, "bf16": 1, "mxfp8": 2}
STATUS = {0: "GDPA_OK", 1: "GDPA_EINVAL", 2: "GDPA_ENOTSUP", 3: "GDPA_EWORKSPACE", 4: "GDPA_EHIP"}

# Every symbol include/gdpa.h declares.
EXPORTS = ["gdpa_abi_version", "gdpa_status_string", "gdpa_workspace_size", "gdpa_fwd",
           "gdpa_fwd_static", "gdpa_fwd_plan_bwd", "gdpa_bwd", "gdpa_bwd_planned", "gdpa_bwd_mx", "gdpa_block_workspace_size", "gdpa_block_fwd",
           "gdpa_block_bwd",
           "gdpa_read_device_error", "gdpa_item_list", "gdpa_profile_start", "gdpa_profile_read",
           "gdpa_profile_stop"]

# kernels selectable by the profiling hook
PROFILE_KERNELS = {"fwd": 0, "dq": 1, "dkdv": 2, "sched": 3, "block_fwd": 4, "block_bwd": 5}


class GdpaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("total_q", ctypes.c_int64),
                ("total_kv", ctypes.c_int64), ("max_q", ctypes.c_int32),
                ("max_kv", ctypes.c_int32), ("act", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("scale", ctypes.c_float), ("bias_buckets", ctypes.c_int32),
                ("window", ctypes.c_int32), ("q_shared", ctypes.c_int32)]


class GdpaBlockProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("total", ctypes.c_int64), ("act", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float), ("block", ctypes.c_int32),
                ("rotary", ctypes.c_int32), ("rope_base", ctypes.c_float)]


class GdpaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


_lib = None


def load():
    """Load libgdpa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(GdpaProblem)
    lib.gdpa_abi_version.restype = ctypes.c_int32
    lib.gdpa_abi_version.argtypes = []
    lib.gdpa_status_string.restype = ctypes.c_char_p
    lib.gdpa_status_string.argtypes = [ctypes.c_int32]
    lib.gdpa_workspace_size.restype = ctypes.c_int32
    lib.gdpa_workspace_size.argtypes = [P, ctypes.c_int32, ctypes.POINTER(sz)]
    lib.gdpa_fwd.restype = ctypes.c_int32
    lib.gdpa_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_fwd_static.restype = ctypes.c_int32
    lib.gdpa_fwd_static.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdpa_bwd_mx.restype = ctypes.c_int32
    lib.gdpa_bwd_mx.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, sz, vp]
    BP = ctypes.POINTER(GdpaBlockProblem)
    lib.gdpa_block_workspace_size.restype = ctypes.c_int32
    lib.gdpa_block_workspace_size.argtypes = [BP, ctypes.POINTER(sz)]
    lib.gdpa_block_fwd.restype = ctypes.c_int32
    lib.gdpa_block_fwd.argtypes = [BP, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_block_bwd.restype = ctypes.c_int32
    lib.gdpa_block_bwd.argtypes = [BP, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_bwd.restype = ctypes.c_int32
    lib.gdpa_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_bwd_planned.restype = ctypes.c_int32
    lib.gdpa_bwd_planned.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdpa_fwd_plan_bwd.restype = ctypes.c_int32
    lib.gdpa_fwd_plan_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.gdpa_read_device_error.restype = ctypes.c_int32
    lib.gdpa_read_device_error.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32)]
    lib.gdpa_item_list.restype = ctypes.c_int32
    lib.gdpa_item_list.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(sz),
                                   ctypes.POINTER(ctypes.c_int64)]
    lib.gdpa_profile_start.restype = ctypes.c_int32
    lib.gdpa_profile_start.argtypes = [ctypes.c_int32]
    lib.gdpa_profile_read.restype = ctypes.c_int32
    lib.gdpa_profile_read.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                      ctypes.POINTER(ctypes.c_double)]
    lib.gdpa_profile_stop.restype = ctypes.c_int32
    lib.gdpa_profile_stop.argtypes = []
    if lib.gdpa_abi_version() != 3:
        raise RuntimeError("libgdpa.so ABI version mismatch")
    _lib = lib
    return lib


def problem(B, H, D, total_q, total_kv, *, dtype="bf16", act="softmax", causal=False,
            scale=None, bias_buckets=0, max_q=0, max_kv=0, window=0, q_shared=False):
    if scale is None:
        scale = D ** -0.5
    return GdpaProblem(B=B, H=H, D=D, dtype=DTYPE[dtype], total_q=total_q, total_kv=total_kv,
                       max_q=max_q, max_kv=max_kv, act=ACT[act], causal=int(bool(causal)),
                       scale=float(scale), bias_buckets=bias_buckets, window=int(window),
                       q_shared=int(bool(q_shared)))


def workspace_size(prob, for_bwd=False):
    lib = load()
    n = ctypes.c_size_t(0)
    st = lib.gdpa_workspace_size(ctypes.byref(prob), int(bool(for_bwd)), ctypes.byref(n))
    if st != 0:
        raise GdpaError(st, "gdpa_workspace_size")
    return int(n.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_of(t):
    if t.dtype == torch.float32:
        return "f32"
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.uint8:
        return "mxfp8"
    raise TypeError(f"unsupported element type {t.dtype}")


def _workspace(nbytes, device):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def fwd(q, k, v, q_offsets, kv_offsets, *, act="softmax", causal=False, scale=None, bias=None,
        q_scale=None, k_scale=None, v_scale=None, max_q=0, max_kv=0, out=None, lse=None,
        workspace=None, stream=None, return_lse=True, window=0, q_shared=False, total_q=None,
        plan_bwd=None):
    """Forward over jagged tensors q [total_q, H, D], k/v [total_kv, H, D].

    bf16 / fp32 tensors, or uint8 e4m3 codes with uint8 e8m0 scales [rows, H, D/32] (MX).
    q_shared: q is one block [max_q, H, D] that every sample reads (local query i = row i); the
    output row count total_q (= q_offsets[-1]) then comes from `total_q` or `out`.
    plan_bwd: the backward's workspace (bf16 / fp32): the forward also builds the backward's work
    lists there (gdpa_fwd_plan_bwd), for one bwd(..., workspace=plan_bwd, planned=True).
    Returns (O, lse); lse is None for GDPA activations.
    """
    lib = load()
    rows, H, D = q.shape
    if q_shared:
        max_q = rows
        if out is not None:
            total_q = out.shape[0]
        elif total_q is None:
            raise ValueError("q_shared needs total_q or out")
    else:
        total_q = rows
    B = q_offsets.numel() - 1
    dt = _dtype_of(q)
    prob = problem(B, H, D, total_q, k.shape[0], dtype=dt, act=act, causal=causal, scale=scale,
                   bias_buckets=0 if bias is None else bias.shape[1], max_q=max_q, max_kv=max_kv,
                   window=window, q_shared=q_shared)
    out_dtype = torch.float32 if dt == "f32" else torch.bfloat16
    if out is None:
        out = torch.empty((total_q, H, D), dtype=out_dtype, device=q.device)
    if act == "softmax" and return_lse and lse is None:
        lse = torch.empty((total_q, H), dtype=torch.float32, device=q.device)
    if act != "softmax":
        lse = None
    if workspace is None:
        workspace = _workspace(workspace_size(prob, False), q.device)
    if plan_bwd is not None:
        st = lib.gdpa_fwd_plan_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets),
                                   _ptr(kv_offsets), _ptr(bias), _ptr(out), _ptr(lse),
                                   _ptr(workspace), workspace.numel(), _ptr(plan_bwd),
                                   plan_bwd.numel(), _stream(stream))
        if st != 0:
            raise GdpaError(st, "gdpa_fwd_plan_bwd")
        return out, lse
    st = lib.gdpa_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale),
                      _ptr(k_scale), _ptr(v_scale), _ptr(q_offsets), _ptr(kv_offsets),
                      _ptr(bias), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                      _stream(stream))
    if st != 0:
        raise GdpaError(st, "gdpa_fwd")
    return out, lse


STATIC_SCRATCH_BYTES = 48 << 20  # GDPA_STATIC_SCRATCH_BYTES


def fwd_static(q, k, v, q_offsets, kv_offsets, out, lse=None, *, act="softmax", causal=False,
               scale=None, bias=None, q_scale=None, k_scale=None, v_scale=None, max_q=0,
               max_kv=0, stream=None, window=0):
    """gdpa_fwd_static: the forward with the library's fixed per-GPU scratch instead of a
    workspace. The caller passes the outputs (out [total_q, H, D]; lse [total_q, H] for softmax,
    or None); nothing is allocated here or in the library. Calls on one GPU must not overlap in
    time (they share the scratch)."""
    lib = load()
    total_q, H, D = q.shape
    prob = problem(q_offsets.numel() - 1, H, D, total_q, k.shape[0], dtype=_dtype_of(q), act=act,
                   causal=causal, scale=scale, bias_buckets=0 if bias is None else bias.shape[1],
                   max_q=max_q, max_kv=max_kv, window=window)
    st = lib.gdpa_fwd_static(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale),
                             _ptr(k_scale), _ptr(v_scale), _ptr(q_offsets), _ptr(kv_offsets),
                             _ptr(bias), _ptr(out), _ptr(lse if act == "softmax" else None),
                             _stream(stream))
    if st != 0:
        raise GdpaError(st, "gdpa_fwd_static")
    return out, lse


def bwd(q, k, v, o, do, lse, q_offsets, kv_offsets, *, act="softmax", causal=False, scale=None,
        bias=None, max_q=0, max_kv=0, workspace=None, stream=None, grads=None, window=0,
        q_shared=False, q_scale=None, k_scale=None, v_scale=None, planned=False):
    """Backward of sum(do * O). Returns (dQ, dK, dV, dbias or None).

    planned: `workspace` holds the work lists a fwd(..., plan_bwd=workspace) on the same problem
    and offsets built (gdpa_bwd_planned: no scheduler launch here).

    q_shared: q (and so dQ) is one block [max_q, H, D] read by every sample; dQ is the sum of
    the samples' gradients. total_q is then do's row count.
    MX-fp8 inputs (uint8 codes with q_scale/k_scale/v_scale) go to gdpa_bwd_mx; the gradients
    are bf16.
    """
    if planned and workspace is None:
        raise ValueError("planned needs the workspace the forward planned")
    lib = load()
    total_q, H, D = q.shape
    if q_shared:
        max_q, total_q = q.shape[0], do.shape[0]
    B = q_offsets.numel() - 1
    dt = _dtype_of(q)
    nb = 0 if bias is None else bias.shape[1]
    prob = problem(B, H, D, total_q, k.shape[0], dtype=dt, act=act, causal=causal, scale=scale,
                   bias_buckets=nb, max_q=max_q, max_kv=max_kv, window=window, q_shared=q_shared)
    if grads is None:
        gdt = torch.bfloat16 if dt == "mxfp8" else q.dtype
        dq = torch.empty(q.shape, dtype=gdt, device=q.device)
        dk = torch.empty(k.shape, dtype=gdt, device=k.device)
        dv = torch.empty(v.shape, dtype=gdt, device=v.device)
        dbias = torch.empty_like(bias) if bias is not None else None
    else:
        dq, dk, dv, dbias = grads
    if workspace is None:
        workspace = _workspace(workspace_size(prob, True), q.device)
    if dt == "mxfp8":
        st = lib.gdpa_bwd_mx(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale),
                             _ptr(k_scale), _ptr(v_scale), _ptr(o), _ptr(do), _ptr(lse),
                             _ptr(q_offsets), _ptr(kv_offsets), _ptr(bias), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(dbias), _ptr(workspace), workspace.numel(),
                             _stream(stream))
        if st != 0:
            raise GdpaError(st, "gdpa_bwd_mx")
        return dq, dk, dv, dbias
    if planned and workspace is None:
        raise ValueError("planned needs the workspace the forward planned")
    fn = lib.gdpa_bwd_planned if planned else lib.gdpa_bwd
    st = fn(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
            _ptr(q_offsets), _ptr(kv_offsets), _ptr(bias), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(dbias), _ptr(workspace), workspace.numel(), _stream(stream))
    if st != 0:
        raise GdpaError(st, "gdpa_bwd_planned" if planned else "gdpa_bwd")
    return dq, dk, dv, dbias


def block_problem(B, H, D, total, *, act="softmax", causal=False, scale=None, block=64,
                  rotary=True, rope_base=10000.0, dtype="bf16"):
    if scale is None:
        scale = D ** -0.5
    return GdpaBlockProblem(B=B, H=H, D=D, dtype=DTYPE[dtype], total=total, act=ACT[act],
                            causal=int(bool(causal)), scale=float(scale), block=block,
                            rotary=int(bool(rotary)), rope_base=float(rope_base))


def block_workspace_size(prob):
    n = ctypes.c_size_t(0)
    st = load().gdpa_block_workspace_size(ctypes.byref(prob), ctypes.byref(n))
    if st != 0:
        raise GdpaError(st, "gdpa_block_workspace_size")
    return int(n.value)


def _block_prob(q, offsets, act, causal, scale, block, rotary, rope_base):
    total, H, D = q.shape
    return block_problem(offsets.numel() - 1, H, D, total, act=act, causal=causal, scale=scale,
                         block=block, rotary=rotary, rope_base=rope_base, dtype=_dtype_of(q))


def block_fwd(q, k, v, offsets, *, act="softmax", causal=False, scale=None, block=64,
              rotary=True, rope_base=10000.0, out=None, workspace=None, stream=None):
    """Block-aligned attention with rotary embeddings over jagged q/k/v [total, H, D] (one
    offsets array). Returns O."""
    prob = _block_prob(q, offsets, act, causal, scale, block, rotary, rope_base)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = _workspace(block_workspace_size(prob), q.device)
    st = load().gdpa_block_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                               _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    if st != 0:
        raise GdpaError(st, "gdpa_block_fwd")
    return out


def block_bwd(q, k, v, do, offsets, *, act="softmax", causal=False, scale=None, block=64,
              rotary=True, rope_base=10000.0, grads=None, workspace=None, stream=None):
    """Backward of sum(do * O) for block_fwd. Returns (dQ, dK, dV)."""
    prob = _block_prob(q, offsets, act, causal, scale, block, rotary, rope_base)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    if workspace is None:
        workspace = _workspace(block_workspace_size(prob), q.device)
    st = load().gdpa_block_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                               _ptr(offsets), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                               workspace.numel(), _stream(stream))
    if st != 0:
        raise GdpaError(st, "gdpa_block_bwd")
    return dq, dk, dv


def read_device_error(workspace, stream=None):
    lib = load()
    err = ctypes.c_int32(0)
    st = lib.gdpa_read_device_error(_ptr(workspace), _stream(stream), ctypes.byref(err))
    if st != 0:
        raise GdpaError(st, "gdpa_read_device_error")
    return int(err.value)


def workspace_header(workspace):
    """Scheduler counters of the last call that used this workspace (diagnostics; synchronises).

    Keys: error, items, items2 (forward / dQ list, dK/dV list), split, split2 (tiles split into
    chunks), chunk, chunk2 (inner tiles per chunk; 0 when splitting is off), die_items,
    die_items2 (per die, the items placed there as their own group's, before the surplus of
    longer dies fills shorter ones).
    """
    torch.cuda.synchronize(workspace.device)
    w = workspace[:92].view(torch.int32).cpu().tolist()
    d = dict(zip(["error", "items", "items2", "split", "split2", "chunk", "chunk2"], w[:7]))
    d["die_items"], d["die_items2"] = w[7:15], w[15:23]
    return d


def item_list(prob, workspace, for_bwd=False, which=0):
    """The scheduler's work items of the last call that used `workspace` (diagnostics;
    synchronises): an int32 array [n, 12] of (sample, tile, head, canonical tile, lo, hi, slot,
    chunk, first query row, query length, first key row, key length) in list order."""
    off = ctypes.c_size_t(0)
    cap = ctypes.c_int64(0)
    st = load().gdpa_item_list(ctypes.byref(prob), int(bool(for_bwd)), int(which),
                               ctypes.byref(off), ctypes.byref(cap))
    if st != 0:
        raise GdpaError(st, "gdpa_item_list")
    n = workspace_header(workspace)["items2" if which else "items"]
    assert 0 <= n <= cap.value
    o = int(off.value)
    return workspace[o:o + 48 * n].view(torch.int32).view(n, 12).cpu().numpy()


def profile_start(kernels):
    """Bracket every launch of the given kernels ("fwd", "dq", "dkdv", "sched") with HIP events."""
    mask = 0
    for k in kernels:
        mask |= 1 << PROFILE_KERNELS[k]
    st = load().gdpa_profile_start(mask)
    if st != 0:
        raise GdpaError(st, "gdpa_profile_start")


def profile_read(kernel):
    """(launches timed, summed duration in ms) of one kernel since profile_start."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    st = load().gdpa_profile_read(PROFILE_KERNELS[kernel], ctypes.byref(n), ctypes.byref(ms))
    if st != 0:
        raise GdpaError(st, "gdpa_profile_read")
    return int(n.value), float(ms.value)


def profile_stop():
    load().gdpa_profile_stop()

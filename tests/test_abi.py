"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and rejects
bad arguments with a status before touching the GPU (no compute call runs here)."""
import ctypes
import os
import re

import pytest

from jagged_attention_recommendation_amd import gdpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "gdpa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|const char\*)\s+(gdpa_\w+)\(", src, re.M)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(gdpa.EXPORTS)


def test_library_exports_every_symbol():
    lib = gdpa.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.gdpa_abi_version() == 3
    assert lib.gdpa_status_string(0) == b"ok"


def test_problem_struct_layout():
    assert ctypes.sizeof(gdpa.GdpaProblem) == 64
    assert gdpa.GdpaProblem.total_q.offset == 16
    assert gdpa.GdpaProblem.scale.offset == 48
    assert gdpa.GdpaProblem.window.offset == 56
    assert gdpa.GdpaProblem.q_shared.offset == 60


def test_workspace_size_validation():
    ok = gdpa.problem(4, 2, 64, 100, 100)
    assert gdpa.workspace_size(ok) >= 256
    # a bias table adds its partial rows (D = 128: the same lists split with and without one)
    assert gdpa.workspace_size(gdpa.problem(4, 2, 128, 100, 100, bias_buckets=16), True) > \
        gdpa.workspace_size(gdpa.problem(4, 2, 128, 100, 100), True)
    with pytest.raises(gdpa.GdpaError) as e:
        gdpa.workspace_size(gdpa.problem(4, 2, 48, 100, 100))
    assert e.value.status == 2  # D = 48 unsupported
    with pytest.raises(gdpa.GdpaError) as e:
        gdpa.workspace_size(gdpa.problem(-1, 2, 64, 100, 100))
    assert e.value.status == 1
    # the MX backward's workspace holds the dequantised Q, K, V and the bf16 backward's own
    mx = gdpa.workspace_size(gdpa.problem(4, 2, 128, 100, 100, dtype="mxfp8"), True)
    bf = gdpa.workspace_size(gdpa.problem(4, 2, 128, 100, 100, dtype="bf16"), True)
    assert mx >= bf + 3 * 100 * 2 * 128 * 2


def test_window_validation():
    """A sliding window needs causal attention on the fp32 or bf16 kernels (not MX); a negative
    window is an argument error."""
    for D in (32, 64, 128):
        for dtype in ("bf16", "f32"):
            ok = gdpa.problem(4, 2, D, 100, 100, causal=True, window=8, dtype=dtype)
            assert gdpa.workspace_size(ok) >= 256 and gdpa.workspace_size(ok, True) >= 256
    for kw, status in [(dict(D=128, causal=True, window=-1), 1),
                       (dict(D=128, causal=False, window=8), 2),
                       (dict(D=64, causal=False, window=8), 2),
                       (dict(D=64, causal=False, window=8, dtype="f32"), 2),
                       (dict(D=128, causal=True, window=8, dtype="mxfp8"), 2)]:
        D = kw.pop("D")
        with pytest.raises(gdpa.GdpaError) as e:
            gdpa.workspace_size(gdpa.problem(4, 2, D, 100, 100, **kw))
        assert e.value.status == status, kw


def test_shared_query_validation():
    """A shared query block needs bf16 or fp32 and max_q >= 1; the backward workspace then holds
    the per-sample fp32 query gradients (total_q * H * D floats) on top of the unshared layout."""
    kw = dict(max_q=32)
    ok = gdpa.problem(8, 2, 64, 256, 1000, q_shared=True, **kw)
    base = gdpa.problem(8, 2, 64, 256, 1000, **kw)
    assert gdpa.workspace_size(ok) == gdpa.workspace_size(base)
    assert gdpa.workspace_size(ok, True) >= gdpa.workspace_size(base, True) + 256 * 2 * 64 * 4
    f32 = gdpa.problem(8, 2, 64, 256, 1000, q_shared=True, dtype="f32", **kw)
    assert gdpa.workspace_size(f32, True) >= 256 * 2 * 64 * 4
    for prob, status in [(gdpa.problem(8, 2, 64, 256, 1000, q_shared=True), 1),  # max_q = 0
                         (gdpa.problem(8, 2, 128, 256, 1000, q_shared=True, dtype="mxfp8", **kw),
                          2)]:
        with pytest.raises(gdpa.GdpaError) as e:
            gdpa.workspace_size(prob)
        assert e.value.status == status
    bad = gdpa.problem(8, 2, 64, 256, 1000, **kw)
    bad.q_shared = 2
    with pytest.raises(gdpa.GdpaError) as e:
        gdpa.workspace_size(bad)
    assert e.value.status == 1


def test_fwd_rejects_host_checkable_errors_without_launching():
    lib = gdpa.load()
    p = gdpa.problem(2, 1, 32, 10, 10)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    big = 1 << 30
    # null offsets
    st = lib.gdpa_fwd(ctypes.byref(p), fake, fake, fake, None, None, None, None, None, None,
                      fake, fake, fake, big, None)
    assert st == 1
    # misaligned Q
    st = lib.gdpa_fwd(ctypes.byref(p), ctypes.c_void_p(0x1002), fake, fake, None, None, None,
                      fake, fake, None, fake, fake, fake, big, None)
    assert st == 1
    # workspace too small
    st = lib.gdpa_fwd(ctypes.byref(p), fake, fake, fake, None, None, None, fake, fake, None,
                      fake, fake, fake, 16, None)
    assert st == 3
    # bias pointer without bias buckets
    st = lib.gdpa_fwd(ctypes.byref(p), fake, fake, fake, None, None, None, fake, fake, fake,
                      fake, fake, fake, big, None)
    assert st == 1
    # scales on a non-MX problem
    st = lib.gdpa_fwd(ctypes.byref(p), fake, fake, fake, fake, None, None, fake, fake, None,
                      fake, fake, fake, big, None)
    assert st == 1


def test_fwd_plan_bwd_rejects_host_checkable_errors_without_launching():
    lib = gdpa.load()
    p = gdpa.problem(2, 1, 32, 10, 10)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    big = 1 << 30
    args = lambda bws, bbytes, ws_bytes=big: (ctypes.byref(p), fake, fake, fake, fake, fake, None,
                                              fake, fake, fake, ws_bytes, bws, bbytes, None)
    assert lib.gdpa_fwd_plan_bwd(*args(None, big)) == 1                     # no backward workspace
    assert lib.gdpa_fwd_plan_bwd(*args(ctypes.c_void_p(0x1008), big)) == 1  # misaligned
    assert lib.gdpa_fwd_plan_bwd(*args(fake, 16)) == 3                      # too small
    assert lib.gdpa_fwd_plan_bwd(*args(fake, big, 16)) == 3                 # forward's too small
    assert lib.gdpa_fwd_plan_bwd(*args(fake, big)) == 1                     # same workspace twice
    pm = gdpa.problem(2, 1, 128, 10, 10, dtype="mxfp8")
    st = lib.gdpa_fwd_plan_bwd(ctypes.byref(pm), fake, fake, fake, fake, fake, None, fake, fake,
                               fake, big, fake, big, None)
    assert st == 2  # MX problems have no planned backward
    # the planned backward validates like gdpa_bwd: null offsets, workspace too small
    st = lib.gdpa_bwd_planned(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None,
                              None, fake, fake, fake, None, fake, big, None)
    assert st == 1
    st = lib.gdpa_bwd_planned(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                              None, fake, fake, fake, None, fake, 16, None)
    assert st == 3
    # valid arguments on a workspace that no gdpa_fwd_plan_bwd planned: refused before any launch
    st = lib.gdpa_bwd_planned(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                              None, fake, fake, fake, None, fake, big, None)
    assert st == 1


def test_block_problem_validation():
    """Block-aligned attention: the struct matches the header's layout (48 bytes), and argument
    errors are reported without any launch."""
    import ctypes
    assert ctypes.sizeof(gdpa.GdpaBlockProblem) == 48
    ok = gdpa.block_problem(3, 2, 128, 500)
    assert gdpa.block_workspace_size(ok) >= 256
    bad = [(dict(D=64), 2), (dict(dtype="f32"), 2), (dict(block=32), 2), (dict(scale=-1.0), 2),
           (dict(rope_base=1.0), 1), (dict(act="nope"), None)]
    for kw, status in bad:
        if status is None:
            continue
        args = dict(B=3, H=2, D=128, total=500)
        args.update({k: v for k, v in kw.items() if k in ("B", "H", "D", "total")})
        p = gdpa.block_problem(args["B"], args["H"], args["D"], args["total"],
                               **{k: v for k, v in kw.items() if k not in args})
        with pytest.raises(gdpa.GdpaError) as e:
            gdpa.block_workspace_size(p)
        assert e.value.status == status, kw
    p = gdpa.block_problem(3, 2, 128, 500)
    p.act = 7
    with pytest.raises(gdpa.GdpaError) as e:
        gdpa.block_workspace_size(p)
    assert e.value.status == 1


def test_bwd_mx_rejects_host_checkable_errors_without_launching():
    """gdpa_bwd_mx checks every argument (its own and those of the bf16 backward it runs after
    the dequantisation) before anything is enqueued; gdpa_bwd refuses MX problems."""
    lib = gdpa.load()
    p = gdpa.problem(2, 1, 128, 10, 10, dtype="mxfp8")
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    big = 1 << 30
    args = [fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, None, fake, fake,
            fake, None, fake, big, None]
    bad = list(args)
    bad[7] = None  # dO
    assert lib.gdpa_bwd_mx(ctypes.byref(p), *bad) == 1
    bad = list(args)
    bad[3] = None  # q_scale
    assert lib.gdpa_bwd_mx(ctypes.byref(p), *bad) == 1
    bad = list(args)
    bad[17] = 64  # workspace too small
    assert lib.gdpa_bwd_mx(ctypes.byref(p), *bad) == 3
    bad = list(args)
    bad[0] = ctypes.c_void_p(0x1004)  # misaligned codes
    assert lib.gdpa_bwd_mx(ctypes.byref(p), *bad) == 1
    pb = gdpa.problem(2, 1, 128, 10, 10, dtype="bf16")
    assert lib.gdpa_bwd_mx(ctypes.byref(pb), *args) == 1  # not an MX problem
    assert lib.gdpa_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, None,
                        fake, fake, fake, None, fake, big, None) == 2

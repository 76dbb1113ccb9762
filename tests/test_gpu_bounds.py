"""Canary guards: no kernel writes outside the buffers it is given.

Every output (O, lse, dQ, dK, dV, dbias) and both workspaces are carved out of larger buffers
filled with a byte pattern; after the forward and the backward the guard bytes before and after
each buffer must be unchanged, and the outputs must still match the fp64 oracle. The problems
cover ragged tails (lengths one below, at and above the tile sizes), empty samples, split tiles,
a sliding window, a shared query block and every element type.
"""
import numpy as np
import pytest
import torch

import oracle
from jagged_attention_recommendation_amd import inputs
from parity_util import assert_close, assert_lse_close, live_rows, to_device
from parity_util import host_f64 as host
from test_gpu_bwd import assert_dbias_close

pytestmark = pytest.mark.gpu

GUARD = 8192
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from jagged_attention_recommendation_amd import gdpa
    gdpa.load()


class Guarded:
    """Buffers with GUARD bytes of PATTERN on each side."""

    def __init__(self):
        self.bufs = []

    def tensor(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((GUARD + n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, n))
        return buf[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        for k, (buf, n) in enumerate(self.bufs):
            lo, hi = buf[:GUARD], buf[GUARD + n:]
            assert bool((lo == PATTERN).all()), f"{what}: write before buffer {k}"
            assert bool((hi == PATTERN).all()), f"{what}: write past buffer {k}"


def run(p, window=0, backward=True):
    from jagged_attention_recommendation_amd import gdpa
    d = to_device(p)
    g = Guarded()
    nb = 0 if p.bias is None else p.bias.shape[1]
    q_shared = getattr(p, "q_shared", False)
    Qd = d["Q"]
    prob = gdpa.problem(p.B, p.H, p.D, p.total_q, p.total_kv, dtype=p.dtype, act=p.act,
                        causal=p.causal, scale=p.scale, bias_buckets=nb, window=window,
                        q_shared=q_shared, max_q=Qd.shape[0] if q_shared else 0)
    odt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    O = g.tensor((p.total_q, p.H, p.D), odt)
    lse = g.tensor((p.total_q, p.H), torch.float32) if p.act == "softmax" else None
    wf = g.tensor((gdpa.workspace_size(prob, False),), torch.uint8)
    kw = dict(act=p.act, causal=p.causal, scale=p.scale, bias=d["bias"], window=window,
              q_shared=q_shared)
    gdpa.fwd(Qd, d["K"], d["V"], d["q_off"], d["kv_off"], out=O, lse=lse, workspace=wf,
             q_scale=d["q_scale"], k_scale=d["k_scale"], v_scale=d["v_scale"], **kw)
    g.check(f"{p.name} forward")
    if not backward:
        return O, lse, None
    grads = (g.tensor(tuple(Qd.shape), Qd.dtype), g.tensor(tuple(d["K"].shape), odt),
             g.tensor(tuple(d["V"].shape), odt),
             g.tensor((p.H, nb), torch.float32) if nb > 0 else None)
    wb = g.tensor((gdpa.workspace_size(prob, True),), torch.uint8)
    gdpa.bwd(Qd, d["K"], d["V"], O, d["dO"], lse, d["q_off"], d["kv_off"], workspace=wb,
             grads=grads, **kw)
    g.check(f"{p.name} backward")
    return O, lse, grads


def check(p, window=0, backward=True):
    O, lse, grads = run(p, window, backward)
    kind = p.dtype
    Or, lser = oracle.fwd(p.q_off, p.kv_off, *(host(p, n) for n in ("Q", "K", "V")), act=p.act,
                          causal=p.causal, scale=p.scale, window=window,
                          bias=None if p.bias is None else p.bias.astype(np.float64))
    assert_close(O, Or, p.q_off, kind, f"{p.name} O", live_rows(p, "q", window))
    if lse is not None:
        assert_lse_close(lse, lser, f"{p.name} lse")
    if not backward:
        return
    r = oracle.bwd(p.q_off, p.kv_off, *(host(p, n) for n in ("Q", "K", "V", "dO")), act=p.act,
                   causal=p.causal, scale=p.scale, window=window, error_scale=True,
                   bias=None if p.bias is None else p.bias.astype(np.float64))
    gk = "f32" if kind == "f32" else "bf16"
    assert_close(grads[0], r["dQ"], p.q_off, gk, f"{p.name} dQ", live_rows(p, "q", window))
    assert_close(grads[1], r["dK"], p.kv_off, gk, f"{p.name} dK", live_rows(p, "k", window))
    assert_close(grads[2], r["dV"], p.kv_off, gk, f"{p.name} dV", live_rows(p, "k", window))
    if p.bias is not None:
        assert_dbias_close(grads[3], r["dbias"], f"{p.name} dbias", r["dbias_scale"])


EDGE_Q = np.array([1, 63, 64, 65, 127, 128, 129, 0, 5, 200])
EDGE_K = np.array([1, 63, 64, 65, 127, 128, 129, 7, 0, 3])


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("act", ["softmax", "silu"])
def test_edges_bf16(D, act):
    p = inputs.make_problem(f"guard-edges-{D}-{act}", seed=91, H=3, D=D, lq=EDGE_Q, lk=EDGE_K,
                            dtype="bf16", act=act, causal=False, bias_buckets=24)
    check(p)
    pc = inputs.make_problem(f"guard-edges-causal-{D}-{act}", seed=92, H=2, D=D, lq=EDGE_Q,
                             lk=EDGE_Q, dtype="bf16", act=act, causal=True, bias_buckets=24)
    check(pc)


def test_edges_f32():
    p = inputs.make_problem("guard-edges-f32", seed=93, H=2, D=32, lq=EDGE_Q, lk=EDGE_K,
                            dtype="f32", act="gelu_tanh", causal=False, bias_buckets=8)
    check(p)


def test_edges_mx_forward():
    p = inputs.make_problem("guard-edges-mx", seed=94, H=2, D=128, lq=EDGE_Q, lk=EDGE_K,
                            dtype="mxfp8", act="softmax", causal=False, with_grad=False)
    check(p, backward=False)


def test_split_tiles():
    lq, lk = np.array([200, 2100, 33]), np.array([2500, 90, 700])
    p = inputs.make_problem("guard-split", seed=95, H=2, D=128, lq=lq, lk=lk, dtype="bf16",
                            act="softmax", causal=False, bias_buckets=64)
    check(p)


def test_window():
    lq = np.array([900, 40, 129, 9])
    p = inputs.make_problem("guard-window", seed=96, H=2, D=128, lq=lq, lk=lq, dtype="bf16",
                            act="softmax", causal=True, bias_buckets=64)
    check(p, window=100)


def test_shared_queries():
    from test_gpu_shared_q import oracle_shared
    lq = np.array([32, 5, 0, 32, 17])
    lk = np.array([300, 7, 40, 0, 1200])
    p = inputs.make_problem("guard-shared", seed=97, H=2, D=64, lq=lq, lk=lk, dtype="bf16",
                            act="silu", causal=False, shared_q=True)
    p.Q = p.seeds  # the library reads the one block of seed rows
    p.q_shared = True
    O, lse, grads = run(p)
    O_ref, _, rb = oracle_shared(p)
    assert_close(O, O_ref, p.q_off, "bf16", "shared O", live_rows(p, "q"))
    assert_close(grads[0], rb["dQ"], np.array([0, 32]), "bf16", "shared dQ (seeds)")
    assert_close(grads[1], rb["dK"], p.kv_off, "bf16", "shared dK", live_rows(p, "k"))
    assert_close(grads[2], rb["dV"], p.kv_off, "bf16", "shared dV", live_rows(p, "k"))

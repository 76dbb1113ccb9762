"""Parity of the shared query block (PMA seeds): Q and dQ are one [max_q, H, D] block that every
sample reads (local query i = seed row i). O, lse, dK, dV and dbias match the fp64 oracle as in the
other parity tests; dQ matches the oracle's seed gradient (the sum over samples), with the tolerance
block of a dQ element taken as the whole seed block of its head.
"""
import numpy as np
import pytest
import torch

import oracle
from jagged_attention_recommendation_amd import inputs
from parity_util import assert_close, assert_lse_close, live_rows, to_device
from test_gpu_bwd import assert_dbias_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from jagged_attention_recommendation_amd import gdpa
    gdpa.load()


def seeds_dev(p):
    return torch.from_numpy(np.ascontiguousarray(p.seeds).view(np.int16)).view(torch.bfloat16).cuda()


def run_shared(p, headers=False, window=0):
    from jagged_attention_recommendation_amd import gdpa
    d = to_device(p)
    sd = seeds_dev(p)
    kw = dict(act=p.act, causal=p.causal, scale=p.scale, bias=d["bias"], window=window)
    max_q, H, D = p.seeds.shape
    nb = 0 if p.bias is None else p.bias.shape[1]
    prob = gdpa.problem(p.B, H, D, p.total_q, int(p.kv_off[-1]), dtype="bf16", act=p.act,
                        causal=p.causal, scale=p.scale, bias_buckets=nb, max_q=max_q,
                        q_shared=True, window=window)
    wf = torch.empty(gdpa.workspace_size(prob, False), dtype=torch.uint8, device="cuda")
    wb = torch.empty(gdpa.workspace_size(prob, True), dtype=torch.uint8, device="cuda")
    O, lse = gdpa.fwd(sd, d["K"], d["V"], d["q_off"], d["kv_off"], q_shared=True,
                      total_q=p.total_q, workspace=wf, **kw)
    hf = gdpa.workspace_header(wf) if headers else None
    dq, dk, dv, dbias = gdpa.bwd(sd, d["K"], d["V"], O, d["dO"], lse, d["q_off"], d["kv_off"],
                                 q_shared=True, workspace=wb, **kw)
    hb = gdpa.workspace_header(wb) if headers else None
    out = (O, lse, dq, dk, dv, dbias)
    return (out, hf, hb) if headers else out


def head_slice(p, h):
    """The problem restricted to head h (heads are independent), as fp64 oracle inputs."""
    f = lambda which: inputs.as_f64(p, which)[:, h:h + 1]
    bias = None if p.bias is None else p.bias[h:h + 1].astype(np.float64)
    return f("seeds"), f("K"), f("V"), f("dO"), bias


def oracle_shared(p, heads=None, window=0):
    """fp64 oracle outputs of the shared-query problem, for the given heads (all by default),
    concatenated along the head axis."""
    heads = range(p.H) if heads is None else heads
    outs = []
    for h in heads:
        S, K, V, dO, bias = head_slice(p, h)
        kw = dict(act=p.act, causal=p.causal, scale=p.scale, bias=bias, window=window)
        O, lse = oracle.fwd_shared_q(p.q_off, p.kv_off, S, K, V, **kw)
        g = oracle.bwd_shared_q(p.q_off, p.kv_off, S, K, V, dO, error_scale=True, **kw)
        outs.append((O, lse, g))
    cat = lambda xs: np.concatenate(xs, axis=1)
    O = cat([o[0] for o in outs])
    lse = cat([o[1] for o in outs])
    g = {k: cat([o[2][k] for o in outs]) for k in ("dQ", "dK", "dV")}
    if p.bias is not None:
        g["dbias"] = np.concatenate([o[2]["dbias"] for o in outs], axis=0)
        g["dbias_scale"] = np.concatenate([o[2]["dbias_scale"] for o in outs], axis=0)
    return O, lse, g


def check(p, got, heads=None, window=0):
    O, lse, dq, dk, dv, dbias = got
    hs = list(range(p.H)) if heads is None else list(heads)
    O_ref, lse_ref, rb = oracle_shared(p, hs, window)
    sel = lambda t: t[:, hs]
    assert_close(sel(O), O_ref, p.q_off, "bf16", f"{p.name} O", live_rows(p, "q", window))
    if p.act == "softmax":
        assert_lse_close(sel(lse), lse_ref, f"{p.name} lse")
    max_q = p.seeds.shape[0]
    assert dq.shape == (max_q, p.H, p.D)
    assert_close(sel(dq), rb["dQ"], np.array([0, max_q]), "bf16", f"{p.name} dQ (seeds)")
    assert_close(sel(dk), rb["dK"], p.kv_off, "bf16", f"{p.name} dK", live_rows(p, "k", window))
    assert_close(sel(dv), rb["dV"], p.kv_off, "bf16", f"{p.name} dV", live_rows(p, "k", window))
    if p.bias is not None:
        assert_dbias_close(dbias[hs], rb["dbias"], f"{p.name} dbias", rb["dbias_scale"])


def ragged(D, act, nb, causal, seed, B=24, max_q=40, max_k=400, H=3):
    rng = np.random.default_rng(seed)
    lq = rng.integers(0, max_q + 1, B)
    lq[0], lq[1] = max_q, 0
    lk = rng.integers(1, max_k + 1, B)
    lk[2] = 0
    return inputs.make_problem(f"shared_D{D}_{act}_nb{nb}_c{int(causal)}", seed=seed, H=H, D=D,
                               lq=lq, lk=lk, act=act, causal=causal, bias_buckets=nb,
                               shared_q=True)


CASES = [(32, "silu", 0, False), (32, "softmax", 8, True), (64, "silu", 0, False),
         (64, "gelu_tanh", 16, False), (64, "softmax", 0, True), (128, "softmax", 32, False),
         (128, "gelu_tanh", 0, False), (128, "silu", 16, True)]


@pytest.mark.parametrize("D,act,nb,causal", CASES)
def test_shared_query_ragged(D, act, nb, causal):
    p = ragged(D, act, nb, causal, seed=500 + D + nb)
    print(f"[case] {p.name} B={p.B} lq={p.q_off[-1]} lk={p.kv_off[-1]}", flush=True)
    check(p, run_shared(p))


@pytest.mark.parametrize("act,window", [("softmax", 7), ("silu", 24)])
def test_shared_query_with_sliding_window(act, window):
    """The shared block and a causal sliding window together (bf16, D = 128, bias)."""
    p = ragged(128, act, 16, True, seed=650 + window)
    print(f"[case] {p.name} window={window}", flush=True)
    check(p, run_shared(p, window=window), window=window)


@pytest.mark.parametrize("D,act", [(64, "silu"), (128, "softmax"), (32, "gelu_tanh")])
def test_shared_query_split_tiles(D, act):
    """Long key lists with few samples and one head: the dQ and forward tiles are split into
    chunks, whose fp32 per-sample gradients are then summed over samples."""
    p = inputs.make_problem(f"shared_split_D{D}_{act}", seed=600 + D, H=1, D=D,
                            lq=np.array([32, 20, 32]), lk=np.array([7000, 3000, 12]), act=act,
                            shared_q=True)
    print(f"[case] {p.name}", flush=True)
    got, hf, hb = run_shared(p, headers=True)
    assert hf["error"] == 0 and hb["error"] == 0
    assert hf["split"] > 0 and hb["split"] > 0, (hf, hb)
    check(p, got)


def test_shared_query_bitwise_repeatable():
    p = ragged(64, "silu", 16, False, seed=700)
    a = run_shared(p)
    b = run_shared(p)
    for x, y in zip(a, b):
        if x is not None:
            assert torch.equal(x, y)


@pytest.mark.timeout(300)
def test_shared_query_pma_workload_full_size():
    """The PMA workload at its full size (B = 512, H = 8, D = 64, 32 seeds, keys ~ lognormal):
    every output of every head against the oracle, and the whole of O, dK and dV bitwise equal
    to the same kernels' outputs on the seeds materialised per sample (same values, same
    order)."""
    from jagged_attention_recommendation_amd import gdpa
    p = inputs.config_problem(4)
    assert p.seeds.shape == (32, 8, 64)
    print(f"[case] {p.name} B={p.B} total_kv={p.kv_off[-1]}", flush=True)
    got = run_shared(p)
    check(p, got)
    d = to_device(p)
    O_mat, _ = gdpa.fwd(d["Q"], d["K"], d["V"], d["q_off"], d["kv_off"], act=p.act,
                        causal=p.causal, scale=p.scale)
    assert torch.equal(got[0], O_mat)
    # dK and dV read the same query values in the same order from either layout
    _, dk_mat, dv_mat, _ = gdpa.bwd(d["Q"], d["K"], d["V"], O_mat, d["dO"], None, d["q_off"],
                                    d["kv_off"], act=p.act, causal=p.causal, scale=p.scale)
    assert torch.equal(got[3], dk_mat) and torch.equal(got[4], dv_mat)


def test_shared_query_sample_longer_than_block_is_a_device_error():
    """A sample with more queries than the shared block is a malformed q_offsets: the device error
    word is set and every kernel of the call skips its work."""
    from jagged_attention_recommendation_amd import gdpa
    p = ragged(64, "silu", 0, False, seed=701, B=4, max_q=16)
    d = to_device(p)
    sd = seeds_dev(p)[:8]  # a block shorter than the longest sample (16)
    prob = gdpa.problem(p.B, p.H, p.D, p.total_q, int(p.kv_off[-1]), act="silu", max_q=8,
                        q_shared=True)
    for for_bwd in (False, True):
        ws = torch.empty(gdpa.workspace_size(prob, for_bwd), dtype=torch.uint8, device="cuda")
        O, _ = gdpa.fwd(sd, d["K"], d["V"], d["q_off"], d["kv_off"], act="silu", q_shared=True,
                        total_q=p.total_q, workspace=None if for_bwd else ws)
        if for_bwd:
            gdpa.bwd(sd, d["K"], d["V"], O, d["dO"], None, d["q_off"], d["kv_off"], act="silu",
                     q_shared=True, workspace=ws)
        assert gdpa.read_device_error(ws) == 1


@pytest.mark.parametrize("D,act,nb,causal", [(32, "silu", 0, False), (64, "softmax", 8, True),
                                             (128, "gelu_tanh", 0, False)])
def test_shared_query_f32(D, act, nb, causal):
    """fp32 kernels with the shared seed block: Q read at row i for every sample, per-sample
    fp32 query gradients summed over samples in a fixed order (kept in fp32)."""
    from jagged_attention_recommendation_amd import gdpa
    rng = np.random.default_rng(900 + D)
    lq = rng.integers(0, 21, 10)
    lq[0] = 20
    lk = rng.integers(1, 150, 10)
    p = inputs.make_problem(f"shared_f32_D{D}_{act}", seed=900 + D, H=2, D=D, lq=lq, lk=lk,
                            dtype="f32", act=act, causal=causal, bias_buckets=nb, shared_q=True)
    d = to_device(p)
    sd = torch.from_numpy(np.ascontiguousarray(p.seeds)).cuda()
    kw = dict(act=p.act, causal=p.causal, scale=p.scale, bias=d["bias"])
    O, lse = gdpa.fwd(sd, d["K"], d["V"], d["q_off"], d["kv_off"], q_shared=True,
                      total_q=p.total_q, **kw)
    dq, dk, dv, dbias = gdpa.bwd(sd, d["K"], d["V"], O, d["dO"], lse, d["q_off"], d["kv_off"],
                                 q_shared=True, **kw)
    torch.cuda.synchronize()
    assert O.dtype == torch.float32 and dq.dtype == torch.float32
    O_ref, lse_ref, rb = oracle_shared(p)
    assert_close(O, O_ref, p.q_off, "f32", f"{p.name} O", live_rows(p, "q"))
    if p.act == "softmax":
        assert_lse_close(lse, lse_ref, f"{p.name} lse")
    assert_close(dq, rb["dQ"], np.array([0, p.seeds.shape[0]]), "f32", f"{p.name} dQ (seeds)")
    assert_close(dk, rb["dK"], p.kv_off, "f32", f"{p.name} dK", live_rows(p, "k"))
    assert_close(dv, rb["dV"], p.kv_off, "f32", f"{p.name} dV", live_rows(p, "k"))

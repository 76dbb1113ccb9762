"""Block-aligned attention with rotary embeddings (gdpa_block_fwd / gdpa_block_bwd) against the
fp64 oracle's block_fwd / block_bwd.

The variant of page "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
Foundation Model", block-attention paragraph: fixed 64-token blocks per sample, each attending
within itself, Q and K rotated at their sample positions, the rotation's backward applied to the
fp32 gradients. Cases: every activation, causal and not, rotary on and off, ragged samples whose
last block is short (1, 63, 64, 65, ... tokens), an empty sample, positions up to 20,000, the
JFA workload's shapes at full size, guard bytes around every buffer, bitwise repeatability and
malformed offsets.
"""
import numpy as np
import pytest
import torch

import oracle
from jagged_attention_recommendation_amd import inputs
from parity_util import assert_close, host_f64, to_device

pytestmark = pytest.mark.gpu

EDGES = np.array([1, 63, 64, 65, 127, 128, 129, 0, 200, 1000])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from jagged_attention_recommendation_amd import gdpa
    gdpa.load()


def problem(name, seed, lengths, H, act, causal):
    return inputs.make_problem(name, seed=seed, H=H, D=128, lq=lengths, lk=lengths, dtype="bf16",
                               act=act, causal=causal)


def run(p, rotary, outs=None):
    from jagged_attention_recommendation_amd import gdpa
    d = to_device(p)
    kw = dict(act=p.act, causal=p.causal, scale=p.scale, rotary=rotary)
    O = gdpa.block_fwd(d["Q"], d["K"], d["V"], d["q_off"], out=None if outs is None else outs[0],
                       **kw)
    g = gdpa.block_bwd(d["Q"], d["K"], d["V"], d["dO"], d["q_off"],
                       grads=None if outs is None else outs[1:], **kw)
    torch.cuda.synchronize()
    return (O, *g)


def check(p, rotary=True):
    O, dq, dk, dv = run(p, rotary)
    args = (p.q_off, host_f64(p, "Q"), host_f64(p, "K"), host_f64(p, "V"))
    kw = dict(act=p.act, causal=p.causal, scale=p.scale, rotary=rotary)
    Or, _ = oracle.block_fwd(*args, **kw)
    r = oracle.block_bwd(*args, host_f64(p, "dO"), **kw)
    live = np.ones(p.total_q, dtype=bool)  # every token attends to itself
    tag = f"{p.name} rotary={rotary}"
    assert_close(O, Or, p.q_off, "bf16", f"{tag} O", live)
    assert_close(dq, r["dQ"], p.q_off, "bf16", f"{tag} dQ", live)
    assert_close(dk, r["dK"], p.q_off, "bf16", f"{tag} dK", live)
    assert_close(dv, r["dV"], p.q_off, "bf16", f"{tag} dV", live)


@pytest.mark.parametrize("act", ["softmax", "gelu_tanh", "silu"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("rotary", [True, False])
def test_edges(act, causal, rotary):
    check(problem(f"block-edges-{act}-{int(causal)}", 1100, EDGES, 2, act, causal), rotary)


def test_long_positions():
    """One sample of 20,000 tokens: rotary angles at positions far past one revolution."""
    check(problem("block-long", 1101, np.array([20000, 3]), 1, "softmax", True))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("act", ["softmax", "silu"])
def test_jfa_workload_shapes(act):
    """B = 64, H = 4, lengths uniform in [1, 2048]: the JFA workload's shapes, whole problem."""
    rng = np.random.default_rng(1102)
    lengths = rng.integers(1, 2049, size=64)
    check(problem(f"block-jfa-{act}", 1102, lengths, 4, act, True))


def test_guard_bytes():
    from test_gpu_bounds import Guarded
    p = problem("block-guard", 1103, EDGES, 3, "softmax", True)
    g = Guarded()
    shape = (p.total_q, p.H, p.D)
    outs = tuple(g.tensor(shape, torch.bfloat16) for _ in range(4))
    run(p, True, outs)
    g.check("block kernels")
    ref = run(p, True)
    for x, y in zip(outs, ref):
        assert torch.equal(x, y)


def test_bitwise_repeatable():
    p = problem("block-repeat", 1104, EDGES, 2, "gelu_tanh", False)
    a, b = run(p, True), run(p, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bad_offsets_set_device_error():
    from jagged_attention_recommendation_amd import gdpa
    p = problem("block-bad", 1105, EDGES, 2, "softmax", False)
    d = to_device(p)
    bad = d["q_off"].clone()
    bad[3] = bad[2] - 1
    prob = gdpa.block_problem(p.B, p.H, p.D, p.total_q)
    ws = torch.empty(gdpa.block_workspace_size(prob), dtype=torch.uint8, device="cuda")
    gdpa.block_fwd(d["Q"], d["K"], d["V"], bad, workspace=ws)
    assert gdpa.read_device_error(ws) == 3  # flagged as both query and key offsets
    gdpa.block_bwd(d["Q"], d["K"], d["V"], d["dO"], d["q_off"], workspace=ws)
    assert gdpa.read_device_error(ws) == 0

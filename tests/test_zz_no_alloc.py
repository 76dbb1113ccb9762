"""gdpa_fwd_static, the forward for callers that cannot allocate: same results as gdpa_fwd.

The entry point takes no workspace; its scratch is the library's fixed per-GPU buffer. Two calls
in a row (the second on a smaller problem, so the buffer holds the first call's leftovers) must
each give exactly the bits gdpa_fwd gives with a fresh workspace, and match the fp64 oracle; a
problem that needs more scratch than the buffer holds is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

from jagged_attention_recommendation_amd import inputs
from parity_util import assert_close, assert_lse_close, live_rows, oracle_fwd, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from jagged_attention_recommendation_amd import gdpa
    gdpa.load()


def both(p):
    """Outputs of gdpa_fwd_static and of gdpa_fwd (fresh workspace) on the same inputs."""
    from jagged_attention_recommendation_amd import gdpa
    d = to_device(p)
    kw = dict(act=p.act, causal=p.causal, scale=p.scale, bias=d["bias"], q_scale=d["q_scale"],
              k_scale=d["k_scale"], v_scale=d["v_scale"])
    odt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    O = torch.full((p.total_q, p.H, p.D), float("nan"), dtype=odt, device="cuda")
    lse = torch.full((p.total_q, p.H), float("nan"), device="cuda") if p.act == "softmax" else None
    gdpa.fwd_static(d["Q"], d["K"], d["V"], d["q_off"], d["kv_off"], O, lse, **kw)
    O_ref, lse_ref = gdpa.fwd(d["Q"], d["K"], d["V"], d["q_off"], d["kv_off"], **kw)
    torch.cuda.synchronize()
    return (O, lse), (O_ref, lse_ref)


def check(p):
    (O, lse), (O_ref, lse_ref) = both(p)
    assert torch.equal(O, O_ref)
    if lse is not None:
        assert torch.equal(lse, lse_ref)
    Or, lser = oracle_fwd(p)
    assert_close(O, Or, p.q_off, p.dtype, f"{p.name} O (static scratch)", live_rows(p, "q"))
    if lse is not None:
        assert_lse_close(lse, lser, f"{p.name} lse (static scratch)")


def test_two_calls_second_smaller():
    # the first call splits long tiles (chunk slots and counters in the scratch); the second,
    # smaller one reuses the buffer with the first call's contents still in it
    lq = np.array([1500, 70, 5, 900])
    big = inputs.make_problem("static-big", seed=801, H=2, D=128, lq=lq, lk=lq, dtype="bf16",
                              act="softmax", causal=True, bias_buckets=600, with_grad=False)
    small = inputs.make_problem("static-small", seed=802, H=2, D=128, lq=np.array([130, 1, 64]),
                                lk=np.array([130, 1, 64]), dtype="bf16", act="softmax",
                                causal=True, bias_buckets=600, with_grad=False)
    check(big)
    check(small)


def test_two_calls_gdpa_and_other_types():
    lq, lk = np.array([200, 2100, 33]), np.array([2500, 90, 700])
    a = inputs.make_problem("static-cross", seed=803, H=2, D=64, lq=lq, lk=lk, dtype="bf16",
                            act="silu", causal=False, with_grad=False)
    b = inputs.make_problem("static-mx", seed=804, H=2, D=128, lq=np.array([65, 9]),
                            lk=np.array([300, 1]), dtype="mxfp8", act="softmax", causal=False,
                            with_grad=False)
    c = inputs.make_problem("static-f32", seed=805, H=1, D=32, lq=np.array([3, 40]),
                            lk=np.array([3, 40]), dtype="f32", act="gelu_tanh", causal=False,
                            with_grad=False)
    for p in (a, b, c):
        check(p)


def test_full_jfa_workload_fits():
    """The JFA workload (B = 64, H = 4, D = 128) runs from the fixed scratch."""
    p = inputs.config_problem(2)
    (O, lse), (O_ref, lse_ref) = both(p)
    assert torch.equal(O, O_ref) and torch.equal(lse, lse_ref)


def test_problem_larger_than_scratch_is_refused():
    from jagged_attention_recommendation_amd import gdpa
    H, D = 64, 128
    total = 4 << 20  # item list alone: 64 heads x 32768 tiles x 32 B > the scratch
    prob = gdpa.problem(1, H, D, total, total)
    assert gdpa.workspace_size(prob, False) > gdpa.STATIC_SCRATCH_BYTES
    lib = gdpa.load()
    import ctypes
    O = torch.empty(16, dtype=torch.uint8, device="cuda")  # never written: the call is refused
    off = torch.zeros(2, dtype=torch.int32, device="cuda")
    st = lib.gdpa_fwd_static(ctypes.byref(prob), O.data_ptr(), O.data_ptr(), O.data_ptr(), None,
                             None, None, off.data_ptr(), off.data_ptr(), None, O.data_ptr(),
                             O.data_ptr(), None)
    assert st == 3  # GDPA_EWORKSPACE

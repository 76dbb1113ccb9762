"""Forward parity: libgdpa.so (HIP, gfx950) against the fp64 oracle on identical inputs."""
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


def run_fwd(p, **kw):
    from jagged_attention_recommendation_amd import gdpa
    d = to_device(p)
    O, lse = gdpa.fwd(d["Q"], d["K"], d["V"], d["q_off"], d["kv_off"], act=p.act,
                      causal=p.causal, scale=p.scale, bias=d["bias"], q_scale=d["q_scale"],
                      k_scale=d["k_scale"], v_scale=d["v_scale"], **kw)
    torch.cuda.synchronize()
    return O, lse


def check_fwd(p, nthreads=None):
    O, lse = run_fwd(p)
    Or, lser = oracle_fwd(p, nthreads=nthreads)
    kind = p.dtype
    err = assert_close(O, Or, p.q_off, kind, f"{p.name} O", live_rows(p, "q"))
    if p.act == "softmax":
        assert_lse_close(lse, lser, f"{p.name} lse")
    return err


def test_config1_full():
    check_fwd(inputs.config_problem(1))


def small(seed, D, act, causal, nb, dtype="bf16", B=5, H=2, lo=1, hi=300, same=True):
    rng = np.random.default_rng(seed)
    lq = rng.integers(lo, hi + 1, size=B)
    lk = lq if same else rng.integers(lo, hi + 1, size=B)
    return inputs.make_problem(f"small-{seed}", seed=seed, H=H, D=D, lq=lq, lk=lk, dtype=dtype,
                               act=act, causal=causal, bias_buckets=nb, with_grad=False)


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("act", ["softmax", "gelu_tanh", "silu"])
@pytest.mark.parametrize("causal,nb,same", [(False, 0, False), (True, 0, True), (True, 48, True),
                                            (False, 40, False)])
def test_bf16_small(D, act, causal, nb, same):
    check_fwd(small(100 + D, D, act, causal, nb, same=same))


@pytest.mark.parametrize("act", ["softmax", "silu"])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_small(act, causal):
    check_fwd(small(7, 64, act, causal, 24, dtype="f32", hi=150))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("act", ["softmax", "gelu_tanh"])
def test_edge_lengths(dtype, act):
    # lengths 1, tile-1, tile, tile+1, an empty query block, an empty key block
    lq = np.array([1, 63, 64, 65, 127, 128, 129, 0, 5, 200])
    lk = np.array([1, 63, 64, 65, 127, 128, 129, 7, 0, 3])
    p = inputs.make_problem("edges", seed=5, H=3, D=32, lq=lq, lk=lk, dtype=dtype, act=act,
                            causal=False, bias_buckets=16, with_grad=False)
    check_fwd(p)
    pc = inputs.make_problem("edges-causal", seed=6, H=1, D=64, lq=lq, lk=lk, dtype=dtype,
                             act=act, causal=True, with_grad=False)
    check_fwd(pc)


def test_single_long_sample_and_h1():
    p = inputs.make_problem("long", seed=9, H=1, D=128, lq=[2048], lk=[2048], act="softmax",
                            causal=True, bias_buckets=4096, with_grad=False)
    check_fwd(p)


def test_config2_reduced():
    check_fwd(inputs.config_problem(2, B=3))


def test_config3_reduced():
    check_fwd(inputs.config_problem(3, B=6))


def test_config4_reduced():
    check_fwd(inputs.config_problem(4, B=24))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("k", [2, 3, 4])
def test_full_config(k):
    """Full-size workload, one launch as the benchmark runs it; every output element of every
    sample is compared with the fp64 oracle (run on all host cores)."""
    p = inputs.config_problem(k)
    O, lse = run_fwd(p)
    Or, lser = oracle_fwd(p)
    assert_close(O, Or, p.q_off, p.dtype, f"config{k} O", live_rows(p, "q"))
    if lse is not None:
        assert_lse_close(lse, lser, f"config{k} lse")


def test_deterministic_repeat():
    p = small(11, 128, "softmax", True, 64)
    a, la = run_fwd(p)
    b, lb = run_fwd(p)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_bad_offsets_set_device_error():
    from jagged_attention_recommendation_amd import gdpa
    p = small(12, 64, "silu", False, 0)
    d = to_device(p)
    bad = d["q_off"].clone()
    bad[2] = bad[1] - 1  # decreasing
    ws = torch.empty(gdpa.workspace_size(gdpa.problem(p.B, p.H, p.D, p.total_q, p.total_kv,
                                                       act="silu"), False),
                     dtype=torch.uint8, device="cuda")
    gdpa.fwd(d["Q"], d["K"], d["V"], bad, d["kv_off"], act="silu", workspace=ws)
    assert gdpa.read_device_error(ws) == 1
    gdpa.fwd(d["Q"], d["K"], d["V"], d["q_off"], d["kv_off"], act="silu", workspace=ws)
    assert gdpa.read_device_error(ws) == 0


# ---------------------------------------------------------------------------------------------
# MX-fp8 (e4m3 data, e8m0 scales per 32 elements along D), forward only, D = 128


@pytest.mark.parametrize("act", ["softmax", "silu", "gelu_tanh"])
@pytest.mark.parametrize("causal,nb", [(True, 0), (False, 0), (True, 64)])
def test_mx_small(act, causal, nb):
    check_fwd(small(300, 128, act, causal, nb, dtype="mxfp8", B=4))


def test_mx_edges():
    lq = np.array([1, 63, 64, 65, 127, 128, 129, 0, 5, 200])
    lk = np.array([1, 63, 64, 65, 127, 128, 129, 7, 0, 3])
    for act in ("softmax", "silu"):
        p = inputs.make_problem("mx-edges", seed=31, H=2, D=128, lq=lq, lk=lk, dtype="mxfp8",
                                act=act, causal=False, with_grad=False)
        check_fwd(p)


@pytest.mark.parametrize("act", ["softmax", "silu"])
def test_config5_reduced(act):
    check_fwd(inputs.config_problem(5, act=act, B=6, seed=2005))


@pytest.mark.timeout(400)
@pytest.mark.parametrize("act", ["softmax", "silu"])
def test_config5_full(act):
    """Full-size MX workload in one launch; every sample (up to 7,824 tokens for this draw) is
    compared element by element with the fp64 oracle on the dequantised inputs."""
    p = inputs.config_problem(5, act=act)
    O, lse = run_fwd(p)
    Og = O.float().cpu().numpy().astype(np.float64)
    lseg = lse.cpu().numpy() if lse is not None else None
    del O, lse
    Or, lser = oracle_fwd(p)
    assert_close(Og, Or, p.q_off, "mxfp8", "config5 O", live_rows(p, "q"))
    if lseg is not None:
        assert_lse_close(lseg, lser, "config5 lse")

"""The parity tolerance's reading of zero rows, checked on the CPU (no GPU involved).

Under a causal mask with fewer queries than keys (top-left aligned), keys past the last query are
reached by no query: their dK and dV rows are exactly zero, and they form no sum. The other rows
carry the rounding of P to bf16 before the product P^T dO. This test simulates that rounding on
the CPU for a causal SiLU sample with 40 queries and 350 keys (D = 128), the shape on which a GPU
dV element exceeded a bound whose rms counted the zero rows, and checks

  * the simulated bf16 result meets the tolerance with the rms taken over the rows that form a
    sum (the parity rule), and its zero rows are exactly zero (the rule requires that of the GPU);
  * counting the zero rows shrinks the rms by sqrt(rows that form a sum / all rows), the factor
    by which the old bound was tighter than the rounding it was meant to cover;
  * rounding P alone moves dV by up to several parts in a thousand of its block rms: errors of
    the size the GPU showed come from that rounding, not from a wrong result.
"""
import numpy as np
import torch

from jagged_attention_recommendation_amd import inputs
from parity_util import TOL, assert_close, block_scale, live_rows, oracle_bwd


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_zero_rows_and_bf16_probability_rounding():
    Lq, Lk, D = 40, 350, 128
    p = inputs.make_problem("causal-short-queries", seed=2024, H=1, D=D, lq=[Lq], lk=[Lk],
                            dtype="bf16", act="silu", causal=True)
    Q, K, dO = (inputs.as_f64(p, n)[:, 0] for n in ("Q", "K", "dO"))
    ref = oracle_bwd(p)["dV"]                                       # [Lk, 1, D]
    # the bf16 pipeline's dV: P = silu(S) in fp32 and rounded to bf16, fp32-exact accumulation
    # of P^T dO, the result rounded to bf16
    S = p.scale * Q @ K.T
    P = np.where(np.tri(Lq, Lk, dtype=bool), _silu(S), 0.0)
    sim = _bf16((_bf16(P).T @ dO))[:, None, :]
    # keys past the last query: exactly zero in the oracle and in the simulation
    assert not ref[Lq:].any() and not sim[Lq:].any()
    assert (ref[:Lq] != 0).any(axis=2).all()
    # the parity rule accepts the simulated rounding
    assert_close(sim, ref, p.kv_off, "bf16", "simulated bf16 dV", live_rows(p, "k"))
    # the rms over all rows is the rms over the live rows times sqrt(live / all)
    rms_live = np.sqrt((ref[:Lq] ** 2).mean())
    rms_all = np.sqrt((ref ** 2).mean())
    np.testing.assert_allclose(rms_all, rms_live * np.sqrt(Lq / Lk), rtol=1e-12)
    assert block_scale(ref, p.kv_off, live_rows(p, "k"))[0, 0] == max(1.0, rms_live)
    assert block_scale(ref, p.kv_off)[0, 0] == max(1.0, rms_live)
    # P's rounding alone moves dV by a few parts in a thousand of the block rms
    err = np.abs(_bf16(P).T @ dO - P.T @ dO)
    assert err.max() > 1e-3 * rms_live
    assert err.max() < TOL["bf16"][0] * rms_live

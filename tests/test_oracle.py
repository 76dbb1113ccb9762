"""Pins for the fp64 oracle: it is checked against library routines, brute force, closed forms,
invariants and finite differences, never against itself or the GPU path.

The torch references below are written here from library primitives (fp64 CPU
``scaled_dot_product_attention``, ``softmax``, ``F.gelu(approximate="tanh")``, ``F.silu``,
``torch.autograd``); they pad every sample to the longest length and carry the jaggedness in an
explicit mask, so "jagged oracle == padded library attention with a mask" is checked too.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from jagged_attention_recommendation_amd import inputs, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------------
# helpers: small random jagged problems and the padded torch reference


def rand_problem(seed, B=3, H=2, D=4, lq=None, lk=None, maxlen=6, nb=0, same=True):
    rng = np.random.default_rng(seed)
    if lq is None:
        lq = rng.integers(1, maxlen + 1, size=B)
    if lk is None:
        lk = lq.copy() if same else rng.integers(1, maxlen + 1, size=B)
    lq, lk = np.asarray(lq), np.asarray(lk)
    qo, ko = inputs.offsets_from_lengths(lq), inputs.offsets_from_lengths(lk)
    Q = rng.standard_normal((qo[-1], H, D))
    K = rng.standard_normal((ko[-1], H, D))
    V = rng.standard_normal((ko[-1], H, D))
    dO = rng.standard_normal((qo[-1], H, D))
    bias = rng.standard_normal((H, nb)) * 0.5 if nb > 0 else None
    return dict(qo=qo, ko=ko, Q=Q, K=K, V=V, dO=dO, bias=bias)


def padded_torch(pb, act, causal, scale, requires_grad=False, window=0):
    """Dense padded reference: [B, H, Lmax, D] tensors, mask carries lengths/causality/window/bias."""
    qo, ko = pb["qo"], pb["ko"]
    B = len(qo) - 1
    H, D = pb["Q"].shape[1:]
    lq, lk = np.diff(qo), np.diff(ko)
    Lq, Lk = max(1, int(lq.max(initial=0))), max(1, int(lk.max(initial=0)))
    Qt = torch.tensor(pb["Q"], dtype=torch.float64, requires_grad=requires_grad)
    Kt = torch.tensor(pb["K"], dtype=torch.float64, requires_grad=requires_grad)
    Vt = torch.tensor(pb["V"], dtype=torch.float64, requires_grad=requires_grad)
    bt = None
    if pb["bias"] is not None:
        bt = torch.tensor(pb["bias"], dtype=torch.float64, requires_grad=requires_grad)

    def pad(X, off, L):
        rows = []
        for b in range(B):
            x = X[off[b]:off[b + 1]]  # [l, H, D]
            x = torch.cat([x, x.new_zeros((L - x.shape[0], H, D))], 0)
            rows.append(x.permute(1, 0, 2))
        return torch.stack(rows)  # [B, H, L, D]

    q, k, v = pad(Qt, qo, Lq), pad(Kt, ko, Lk), pad(Vt, ko, Lk)
    i = torch.arange(Lq)[:, None]
    j = torch.arange(Lk)[None, :]
    valid = torch.zeros(B, 1, Lq, Lk, dtype=torch.bool)
    for b in range(B):
        m = (i < int(lq[b])) & (j < int(lk[b]))
        if causal:
            m = m & (j <= i)
        if window > 0:
            m = m & (j > i - window)
        valid[b, 0] = m
    add = torch.zeros(B, H, Lq, Lk, dtype=torch.float64)
    if bt is not None:
        nb = bt.shape[1]
        idx = (i - j).clamp(0, nb - 1)  # [Lq, Lk]
        add = add + bt[:, idx][None]
    if act == "softmax":
        neg = torch.where(valid, torch.zeros((), dtype=torch.float64),
                          torch.full((), -math.inf, dtype=torch.float64))
        # rows with no valid key would be NaN; the problems here always keep j = 0 valid
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=add + neg, scale=scale)
    else:
        s = scale * torch.matmul(q, k.transpose(-1, -2).contiguous()) + add
        a = F.gelu(s, approximate="tanh") if act == "gelu_tanh" else F.silu(s)
        o = torch.matmul(torch.where(valid, a, torch.zeros_like(a)), v)
    # unpad
    out = []
    for b in range(B):
        out.append(o[b, :, :int(lq[b])].permute(1, 0, 2))
    O = torch.cat(out, 0) if out else torch.zeros(0, H, D, dtype=torch.float64)
    return O, (Qt, Kt, Vt, bt)


def run_oracle_fwd(pb, act, causal, scale, window=0):
    return oracle.fwd(pb["qo"], pb["ko"], pb["Q"], pb["K"], pb["V"], act=act, causal=causal,
                      scale=scale, bias=pb["bias"], nthreads=2, window=window)


def run_oracle_bwd(pb, act, causal, scale, window=0):
    return oracle.bwd(pb["qo"], pb["ko"], pb["Q"], pb["K"], pb["V"], pb["dO"], act=act,
                      causal=causal, scale=scale, bias=pb["bias"], nthreads=2, error_scale=True,
                      window=window)


CASES = [
    # act, causal, nb, same-length
    ("softmax", False, 0, True),
    ("softmax", True, 0, True),
    ("softmax", True, 4, True),    # clamp binds: i - j up to 7 > NB - 1 = 3
    ("softmax", False, 5, False),  # negative i - j clamps to 0; Lq != Lk
    ("gelu_tanh", False, 0, False),
    ("gelu_tanh", True, 6, True),
    ("silu", False, 3, False),
    ("silu", True, 0, True),
]


# ----------------------------------------------------------------------------------------------
# forward


@pytest.mark.parametrize("act,causal,nb,same", CASES)
@pytest.mark.parametrize("seed", [0, 1])
def test_fwd_matches_padded_library_attention(act, causal, nb, same, seed):
    pb = rand_problem(seed, B=3, H=2, D=5, maxlen=8, nb=nb, same=same)
    scale = 0.7
    O, lse = run_oracle_fwd(pb, act, causal, scale)
    Oref, _ = padded_torch(pb, act, causal, scale)
    np.testing.assert_allclose(O, Oref.detach().numpy(), rtol=1e-12, atol=1e-12)


def test_fwd_lse_against_library_logsumexp():
    pb = rand_problem(3, B=3, H=2, D=4, maxlen=7, nb=4)
    scale = 0.9
    _, lse = run_oracle_fwd(pb, "softmax", True, scale)
    # library logsumexp over the valid keys of each row
    for b in range(3):
        for h in range(2):
            q = torch.tensor(pb["Q"][pb["qo"][b]:pb["qo"][b + 1], h])
            k = torch.tensor(pb["K"][pb["ko"][b]:pb["ko"][b + 1], h])
            L = q.shape[0]
            s = scale * q @ k.T
            i = torch.arange(L)[:, None]
            j = torch.arange(k.shape[0])[None, :]
            s = s + torch.tensor(pb["bias"][h])[(i - j).clamp(0, 3)]
            s = torch.where(j <= i, s, torch.full_like(s, -math.inf))
            ref = torch.logsumexp(s, dim=1).numpy()
            np.testing.assert_allclose(lse[pb["qo"][b]:pb["qo"][b + 1], h], ref, rtol=1e-13,
                                       atol=1e-13)


def test_brute_force_pure_python_tiny():
    """A second, loop-only evaluation of the definition on a 2-sample problem."""
    pb = rand_problem(7, B=2, H=1, D=3, lq=[3, 2], lk=[2, 4], nb=2)
    scale = 1.3
    for act in ("softmax", "gelu_tanh", "silu"):
        O, _ = run_oracle_fwd(pb, act, False, scale)
        for b in range(2):
            for i in range(pb["qo"][b + 1] - pb["qo"][b]):
                qi = pb["Q"][pb["qo"][b] + i, 0]
                ks = pb["K"][pb["ko"][b]:pb["ko"][b + 1], 0]
                vs = pb["V"][pb["ko"][b]:pb["ko"][b + 1], 0]
                s = [scale * sum(qi[c] * kk[c] for c in range(3)) + pb["bias"][0][min(max(i - j, 0), 1)]
                     for j, kk in enumerate(ks)]
                if act == "softmax":
                    w = [math.exp(x) for x in s]
                    tot = sum(w)
                    w = [x / tot for x in w]
                elif act == "silu":
                    w = [x / (1 + math.exp(-x)) for x in s]
                else:
                    w = [0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
                         for x in s]
                ref = [sum(w[j] * vs[j][c] for j in range(len(w))) for c in range(3)]
                np.testing.assert_allclose(O[pb["qo"][b] + i, 0], ref, rtol=1e-12, atol=1e-13)


def test_dbias_error_scale_brute_force_tiny():
    """The bias buckets' error scale (a tolerance input, not a result) by a loop-only evaluation:
    scale[h, r]^2 = sum over rows i of m_ir^2 w_i, m_ir = sum of p_ij over the row's pairs in
    bucket r, w_i = sum_j p_ij^2 dp_ij^2 + sum_c do_ic^2 o_ic^2, for softmax; zero for GDPA,
    which has no row term D_i. The Monte-Carlo test below pins what the formula stands for."""
    pb = rand_problem(8, B=2, H=2, D=3, lq=[4, 2], lk=[3, 5], nb=3)
    scale = 0.8
    for causal in (False, True):
        g = run_oracle_bwd(pb, "softmax", causal, scale)
        ref = np.zeros((2, 3))
        for h in range(2):
            for b in range(2):
                q0, k0 = pb["qo"][b], pb["ko"][b]
                for i in range(pb["qo"][b + 1] - q0):
                    js = [j for j in range(pb["ko"][b + 1] - k0) if not causal or j <= i]
                    if not js:
                        continue
                    s = {j: scale * sum(pb["Q"][q0 + i, h, c] * pb["K"][k0 + j, h, c] for c in range(3))
                         + pb["bias"][h][min(max(i - j, 0), 2)] for j in js}
                    mx = max(s.values())
                    w = {j: math.exp(s[j] - mx) for j in js}
                    tot = sum(w.values())
                    pr = {j: w[j] / tot for j in js}
                    wi = 0.0
                    for j in js:
                        dpj = sum(pb["dO"][q0 + i, h, c] * pb["V"][k0 + j, h, c] for c in range(3))
                        wi += pr[j] ** 2 * dpj ** 2
                    for c in range(3):
                        oc = sum(pr[j] * pb["V"][k0 + j, h, c] for j in js)
                        wi += pb["dO"][q0 + i, h, c] ** 2 * oc * oc
                    m = [0.0, 0.0, 0.0]
                    for j in js:
                        m[min(max(i - j, 0), 2)] += pr[j]
                    for r in range(3):
                        ref[h][r] += m[r] ** 2 * wi
        np.testing.assert_allclose(g["dbias_scale"], np.sqrt(ref), rtol=1e-12, atol=1e-14)
        gd = run_oracle_bwd(pb, "gelu_tanh", causal, scale)
        assert np.array_equal(gd["dbias_scale"], np.zeros((2, 3)))


def _perturbed_dbias_spread(pb, causal, scale, trials, seed):
    """Monte-Carlo simulation of a rounded softmax forward feeding the backward's row term.

    Dense numpy, written here from the definition (no oracle call): exact p_ij, dp_ij, o_i per
    row; then, per trial, every probability is multiplied by (1 + eps z_ij) once (the product
    with V sees the same rounded value in every column) and every output element by
    (1 + eps z'_ic), z ~ N(0, 1) independent. D_i is formed from the perturbed output, ds_ij =
    p_ij (dp_ij - D_i) and the bias gradient are formed from it by their definition, and the
    per-bucket standard deviation of the bias gradient over trials is returned in units of eps."""
    rng = np.random.default_rng(seed)
    eps = 1e-6
    qo, ko = pb["qo"], pb["ko"]
    H, D = pb["Q"].shape[1:]
    nb = pb["bias"].shape[1]
    dev = np.zeros((trials, H, nb))
    for b in range(len(qo) - 1):
        Lq, Lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        for h in range(H):
            q = pb["Q"][qo[b]:qo[b + 1], h]
            k = pb["K"][ko[b]:ko[b + 1], h]
            v = pb["V"][ko[b]:ko[b + 1], h]
            do = pb["dO"][qo[b]:qo[b + 1], h]
            ii, jj = np.meshgrid(np.arange(Lq), np.arange(Lk), indexing="ij")
            valid = (jj <= ii) if causal else np.ones((Lq, Lk), bool)
            bucket = np.clip(ii - jj, 0, nb - 1)
            s = scale * q @ k.T + pb["bias"][h][bucket]
            s = np.where(valid, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)                       # [Lq, Lk]
            dp = do @ v.T
            z = rng.standard_normal((trials, Lq, Lk))
            zo = rng.standard_normal((trials, Lq, D))
            o_t = np.einsum("tij,jc->tic", p[None] * (1 + eps * z), v) * (1 + eps * zo)
            D_t = np.einsum("tic,ic->ti", o_t, do)
            D_x = (p * dp).sum(axis=1)                                 # exact row term
            ds_t = p[None] * (dp[None] - D_t[:, :, None])
            ds_x = p * (dp - D_x[:, None])
            diff = np.where(valid[None], ds_t - ds_x[None], 0.0)
            for r in range(nb):
                dev[:, h, r] += diff[:, bucket == r].sum(axis=1)
    return dev.std(axis=0, ddof=1) / eps


@pytest.mark.parametrize("causal", [False, True])
def test_dbias_error_scale_monte_carlo(causal):
    """Pin of the oracle's bias-bucket error scale against a simulation of what it models: the
    standard deviation of each bucket under independent relative perturbations of the forward's
    probabilities (once per pair) and output elements (once per element) matches
    dbias_scale within the sampling error of the estimate. With T trials the sample variance of
    a Gaussian has relative standard deviation sqrt(2 / T) (0.032 at T = 2000); the check allows
    five of those. Short rows make the sum_j p^2 dp^2 term comparable to the sum_c do^2 o^2 term,
    and buckets that take a single diagonal (m_ir < 1) sit beside clamped edge buckets that take
    whole rows (m_ir = 1), so a dropped term or m_ir in place of m_ir^2 moves some bucket far
    outside the bound."""
    pb = rand_problem(31, B=3, H=2, D=5, lq=[7, 3, 9], nb=4)
    pb["bias"] = pb["bias"] * 2.0
    T = 2000
    sim = _perturbed_dbias_spread(pb, causal, 0.7, T, seed=5)
    g = run_oracle_bwd(pb, "softmax", causal, 0.7)["dbias_scale"]
    live = g > 1e-9
    assert live.sum() >= 6
    assert np.array_equal(live, sim > 1e-9)
    ratio = sim[live] ** 2 / g[live] ** 2
    assert np.all(np.abs(ratio - 1.0) <= 5.0 * np.sqrt(2.0 / T)), ratio


@pytest.mark.parametrize("act", ["softmax", "gelu_tanh", "silu"])
def test_sample_permutation_equivariance_is_bitwise(act):
    pb = rand_problem(11, B=5, H=2, D=4, maxlen=7, nb=3, same=False)
    perm = [3, 0, 4, 2, 1]
    lq, lk = np.diff(pb["qo"]), np.diff(pb["ko"])
    qrows = np.concatenate([np.arange(pb["qo"][b], pb["qo"][b + 1]) for b in perm])
    krows = np.concatenate([np.arange(pb["ko"][b], pb["ko"][b + 1]) for b in perm])
    pp = dict(qo=inputs.offsets_from_lengths(lq[perm]), ko=inputs.offsets_from_lengths(lk[perm]),
              Q=pb["Q"][qrows], K=pb["K"][krows], V=pb["V"][krows], dO=pb["dO"][qrows],
              bias=pb["bias"])
    O, lse = run_oracle_fwd(pb, act, False, 0.8)
    Op, lsep = run_oracle_fwd(pp, act, False, 0.8)
    assert np.array_equal(O[qrows], Op)
    assert np.array_equal(lse[qrows], lsep)
    g = run_oracle_bwd(pb, act, False, 0.8)
    gp = run_oracle_bwd(pp, act, False, 0.8)
    assert np.array_equal(g["dQ"][qrows], gp["dQ"])
    assert np.array_equal(g["dK"][krows], gp["dK"])
    assert np.array_equal(g["dV"][krows], gp["dV"])
    np.testing.assert_allclose(g["dbias"], gp["dbias"], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("act", ["softmax", "gelu_tanh", "silu"])
def test_row_permutations_noncausal_no_bias(act):
    pb = rand_problem(5, B=1, H=2, D=4, lq=[6], lk=[7])
    O, _ = run_oracle_fwd(pb, act, False, 0.6)
    rng = np.random.default_rng(0)
    pk = rng.permutation(7)
    pq = rng.permutation(6)
    pp = dict(pb, K=pb["K"][pk], V=pb["V"][pk], Q=pb["Q"][pq])
    Op, _ = run_oracle_fwd(pp, act, False, 0.6)
    np.testing.assert_allclose(Op, O[pq], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------------------------
# closed forms and special cases


def test_softmax_single_key_returns_that_value_row_exactly():
    pb = rand_problem(2, B=3, H=2, D=6, lq=[4, 1, 3], lk=[1, 1, 1], nb=3)
    O, lse = run_oracle_fwd(pb, "softmax", False, 0.5)
    for b in range(3):
        for r in range(pb["qo"][b], pb["qo"][b + 1]):
            assert np.array_equal(O[r], pb["V"][pb["ko"][b]])  # p = 1 exactly
            i = r - pb["qo"][b]
            s = 0.5 * pb["Q"][r] @ pb["K"][pb["ko"][b]].T  # [H,H]; take the diagonal
            for h in range(2):
                ref = 0.5 * np.dot(pb["Q"][r, h], pb["K"][pb["ko"][b], h]) + pb["bias"][h, min(i, 2)]
                assert abs(lse[r, h] - ref) < 1e-13


def test_softmax_zero_queries_give_mean_of_visible_values():
    pb = rand_problem(4, B=2, H=2, D=3, lq=[5, 3], lk=[5, 3])
    pb["Q"][:] = 0.0
    for causal in (False, True):
        O, lse = run_oracle_fwd(pb, "softmax", causal, 1.0)
        for b in range(2):
            vs = pb["V"][pb["ko"][b]:pb["ko"][b + 1]]
            for i in range(pb["qo"][b + 1] - pb["qo"][b]):
                n = i + 1 if causal else len(vs)
                np.testing.assert_allclose(O[pb["qo"][b] + i], vs[:n].mean(axis=0), rtol=1e-13,
                                           atol=1e-14)
                np.testing.assert_allclose(lse[pb["qo"][b] + i], math.log(n), rtol=1e-14)


def test_softmax_rows_sum_to_one():
    pb = rand_problem(6, B=3, H=2, D=4, maxlen=8, nb=3)
    pb["V"][:] = 1.0
    O, _ = run_oracle_fwd(pb, "softmax", True, 1.7)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("act", ["gelu_tanh", "silu"])
def test_gdpa_closed_forms(act):
    f = (lambda x: F.gelu(torch.tensor(x), approximate="tanh").numpy()) if act == "gelu_tanh" else \
        (lambda x: F.silu(torch.tensor(x)).numpy())
    # Lk = 1: o_i = act(s_i0) v_0
    pb = rand_problem(8, B=2, H=2, D=4, lq=[3, 2], lk=[1, 1])
    O, lse = run_oracle_fwd(pb, act, False, 0.9)
    for b in range(2):
        k0 = pb["ko"][b]
        for r in range(pb["qo"][b], pb["qo"][b + 1]):
            for h in range(2):
                s = 0.9 * np.dot(pb["Q"][r, h], pb["K"][k0, h])
                np.testing.assert_allclose(O[r, h], f(s) * pb["V"][k0, h], rtol=1e-13, atol=1e-15)
    assert np.all(lse == 0.0)
    # Q = 0, no bias: act(0) = 0 so O = 0
    pb = rand_problem(9, B=3, H=2, D=4, maxlen=6)
    pb["Q"][:] = 0.0
    O, _ = run_oracle_fwd(pb, act, True, 1.0)
    assert np.all(O == 0.0)
    # linearity in V and V = 1 gives row sums of act(s)
    pb = rand_problem(10, B=3, H=2, D=4, maxlen=6, nb=2)
    O1, _ = run_oracle_fwd(pb, act, True, 1.1)
    p2 = dict(pb, V=-2.5 * pb["V"])
    O2, _ = run_oracle_fwd(p2, act, True, 1.1)
    np.testing.assert_allclose(O2, -2.5 * O1, rtol=1e-13, atol=1e-14)
    p3 = dict(pb, V=np.ones_like(pb["V"]))
    O3, _ = run_oracle_fwd(p3, act, True, 1.1)
    for b in range(3):
        for h in range(2):
            q = pb["Q"][pb["qo"][b]:pb["qo"][b + 1], h]
            k = pb["K"][pb["ko"][b]:pb["ko"][b + 1], h]
            L = len(q)
            i = np.arange(L)[:, None]
            j = np.arange(len(k))[None, :]
            s = 1.1 * q @ k.T + pb["bias"][h][np.clip(i - j, 0, 1)]
            rs = np.where(j <= i, f(s), 0.0).sum(axis=1)
            np.testing.assert_allclose(O3[pb["qo"][b]:pb["qo"][b + 1], h, 0], rs, rtol=1e-12)


def test_empty_rows_and_samples():
    # sample 0 has no keys, sample 1 has no queries, sample 2 is normal
    qo = np.array([0, 3, 3, 5], np.int32)
    ko = np.array([0, 0, 4, 7], np.int32)
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((5, 1, 4))
    K = rng.standard_normal((7, 1, 4))
    V = rng.standard_normal((7, 1, 4))
    dO = rng.standard_normal((5, 1, 4))
    bias = rng.standard_normal((1, 3))
    for act in ("softmax", "silu"):
        O, lse = oracle.fwd(qo, ko, Q, K, V, act=act, bias=bias)
        assert np.all(O[:3] == 0.0)
        if act == "softmax":
            assert np.all(np.isneginf(lse[:3]))
        g = oracle.bwd(qo, ko, Q, K, V, dO, act=act, bias=bias)
        assert np.all(g["dQ"][:3] == 0.0)
        assert np.all(g["dK"][:4] == 0.0) and np.all(g["dV"][:4] == 0.0)  # sample 1's keys
        assert np.isfinite(g["dQ"]).all() and np.isfinite(g["dbias"]).all()


def test_rejects_bad_offsets():
    Q = np.zeros((3, 1, 4))
    with pytest.raises(ValueError):
        oracle.fwd(np.array([0, 2, 1, 3]), np.array([0, 1, 2, 3]), Q, Q, Q)
    with pytest.raises(ValueError):
        oracle.fwd(np.array([1, 2, 3]), np.array([0, 1, 3]), Q, Q, Q)


# ----------------------------------------------------------------------------------------------
# backward


@pytest.mark.parametrize("act,causal,nb,same", CASES)
def test_bwd_matches_torch_autograd(act, causal, nb, same):
    pb = rand_problem(21, B=3, H=2, D=4, maxlen=7, nb=nb, same=same)
    scale = 0.8
    Oref, (Qt, Kt, Vt, bt) = padded_torch(pb, act, causal, scale, requires_grad=True)
    (Oref * torch.tensor(pb["dO"])).sum().backward()
    g = run_oracle_bwd(pb, act, causal, scale)
    np.testing.assert_allclose(g["dQ"], Qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dK"], Kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dV"], Vt.grad.numpy(), rtol=1e-11, atol=1e-12)
    if nb > 0:
        np.testing.assert_allclose(g["dbias"], bt.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("act,causal,nb", [("softmax", True, 3), ("gelu_tanh", False, 2),
                                           ("silu", True, 4), ("softmax", False, 0)])
def test_bwd_finite_differences(act, causal, nb):
    pb = rand_problem(31, B=2, H=2, D=3, maxlen=5, nb=nb, same=False)
    scale = 0.9
    g = run_oracle_bwd(pb, act, causal, scale)
    h = 1e-6

    def loss(p):
        O, _ = run_oracle_fwd(p, act, causal, scale)
        return float((O * p["dO"]).sum())

    for name, key in (("Q", "dQ"), ("K", "dK"), ("V", "dV"), ("bias", "dbias")):
        if pb[name] is None:
            continue
        base = pb[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += h
            minus[idx] -= h
            fd[idx] = (loss(dict(pb, **{name: plus})) - loss(dict(pb, **{name: minus}))) / (2 * h)
        err = np.abs(fd - g[key]) / np.maximum(1.0, np.abs(g[key]))
        assert err.max() < 1e-6, (name, err.max())


@pytest.mark.parametrize("act", ["softmax", "gelu_tanh", "silu"])
@pytest.mark.parametrize("causal", [False, True])
def test_shared_query_gradient_finite_differences(act, causal):
    """Shared query block (PMA seeds): central differences of sum(dO * O) with respect to each seed
    element match the summed query gradient. Samples of different lengths, one empty and one
    shorter than the block, so a seed row used by only some samples is covered."""
    rng = np.random.default_rng(77)
    H, D, max_q = 2, 3, 4
    lq = np.array([4, 2, 0, 3])
    lk = np.array([3, 5, 2, 1])
    q_off, kv_off = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    seeds = rng.standard_normal((max_q, H, D))
    K = rng.standard_normal((kv_off[-1], H, D))
    V = rng.standard_normal((kv_off[-1], H, D))
    dO = rng.standard_normal((q_off[-1], H, D))
    bias = 0.3 * rng.standard_normal((H, 3))
    kw = dict(act=act, causal=causal, scale=0.8, bias=bias)
    g = oracle.bwd_shared_q(q_off, kv_off, seeds, K, V, dO, **kw)
    assert g["dQ"].shape == seeds.shape

    def loss(sd):
        O, _ = oracle.fwd_shared_q(q_off, kv_off, sd, K, V, **kw)
        return float((O * dO).sum())

    h = 1e-6
    fd = np.zeros_like(seeds)
    for idx in np.ndindex(seeds.shape):
        plus, minus = seeds.copy(), seeds.copy()
        plus[idx] += h
        minus[idx] -= h
        fd[idx] = (loss(plus) - loss(minus)) / (2 * h)
    err = np.abs(fd - g["dQ"]) / np.maximum(1.0, np.abs(g["dQ"]))
    assert err.max() < 1e-6, err.max()


def test_shared_query_identical_samples_scale_gradient():
    """B samples with the same keys, values and output gradient: every sample's output is the
    single-sample output, and the seed gradient is exactly B times the single-sample one (up to
    rounding of the sum)."""
    rng = np.random.default_rng(78)
    H, D, Lq, Lk, B = 2, 8, 5, 7, 6
    seeds = rng.standard_normal((Lq, H, D))
    K1, V1 = rng.standard_normal((Lk, H, D)), rng.standard_normal((Lk, H, D))
    dO1 = rng.standard_normal((Lq, H, D))
    q1, k1 = np.array([0, Lq]), np.array([0, Lk])
    qB, kB = np.arange(B + 1) * Lq, np.arange(B + 1) * Lk
    for act in ("softmax", "silu"):
        O1, _ = oracle.fwd(q1, k1, seeds, K1, V1, act=act)
        g1 = oracle.bwd(q1, k1, seeds, K1, V1, dO1, act=act)
        OB, _ = oracle.fwd_shared_q(qB, kB, seeds, np.tile(K1, (B, 1, 1)), np.tile(V1, (B, 1, 1)),
                                    act=act)
        gB = oracle.bwd_shared_q(qB, kB, seeds, np.tile(K1, (B, 1, 1)), np.tile(V1, (B, 1, 1)),
                                 np.tile(dO1, (B, 1, 1)), act=act)
        np.testing.assert_array_equal(OB, np.tile(O1, (B, 1, 1)))
        np.testing.assert_allclose(gB["dQ"], B * g1["dQ"], rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(gB["dK"], np.tile(g1["dK"], (B, 1, 1)))


def test_shared_query_unused_rows_have_zero_gradient():
    """Seed rows that no sample reaches (every Lq_b shorter than the block) get a zero gradient;
    a single sample that uses the whole block reproduces the plain backward."""
    rng = np.random.default_rng(79)
    H, D = 1, 4
    seeds = rng.standard_normal((6, H, D))
    q_off, kv_off = np.array([0, 2, 5]), np.array([0, 4, 9])
    K, V = rng.standard_normal((9, H, D)), rng.standard_normal((9, H, D))
    dO = rng.standard_normal((5, H, D))
    g = oracle.bwd_shared_q(q_off, kv_off, seeds, K, V, dO, act="gelu_tanh")
    assert (g["dQ"][3:] == 0).all() and (g["dQ"][:3] != 0).any()
    dO6 = rng.standard_normal((6, H, D))
    one = oracle.bwd_shared_q(np.array([0, 6]), np.array([0, 4]), seeds, K[:4], V[:4], dO6,
                              act="softmax")
    plain = oracle.bwd(np.array([0, 6]), np.array([0, 4]), seeds, K[:4], V[:4], dO6, act="softmax")
    np.testing.assert_array_equal(one["dQ"], plain["dQ"])


def test_softmax_backward_invariants():
    pb = rand_problem(41, B=4, H=3, D=5, maxlen=9, nb=6, same=False)
    for causal in (False, True):
        g = run_oracle_bwd(pb, "softmax", causal, 0.7)
        O, _ = run_oracle_fwd(pb, "softmax", causal, 0.7)
        # sum_j ds_ij = 0 per row => the bias gradient sums to zero per head
        np.testing.assert_allclose(g["dbias"].sum(axis=1), 0.0, atol=1e-12)
        # D_i = <do_i, o_i>
        np.testing.assert_allclose(g["D"], (pb["dO"] * O).sum(axis=2), rtol=1e-12, atol=1e-13)
        # sum_j dv_j = sum_i do_i per (sample, head) (every row sees at least one key here)
        for b in range(4):
            sdv = g["dV"][pb["ko"][b]:pb["ko"][b + 1]].sum(axis=0)
            sdo = pb["dO"][pb["qo"][b]:pb["qo"][b + 1]].sum(axis=0)
            np.testing.assert_allclose(sdv, sdo, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# sliding window (causal, W most recent keys)

WINDOW_CASES = [("softmax", 3, 2), ("softmax", 0, 1), ("gelu_tanh", 4, 3), ("silu", 0, 2)]


@pytest.mark.parametrize("act,nb,window", WINDOW_CASES)
def test_window_fwd_bwd_match_padded_library_attention(act, nb, window):
    """The window is one more mask term of the padded library reference (forward and autograd)."""
    pb = rand_problem(51, B=3, H=2, D=4, maxlen=9, nb=nb, same=False)
    scale = 0.8
    O, _ = run_oracle_fwd(pb, act, True, scale, window)
    Oref, (Qt, Kt, Vt, bt) = padded_torch(pb, act, True, scale, requires_grad=True, window=window)
    np.testing.assert_allclose(O, Oref.detach().numpy(), rtol=1e-12, atol=1e-12)
    (Oref * torch.tensor(pb["dO"])).sum().backward()
    g = run_oracle_bwd(pb, act, True, scale, window)
    np.testing.assert_allclose(g["dQ"], Qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dK"], Kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dV"], Vt.grad.numpy(), rtol=1e-11, atol=1e-12)
    if nb > 0:
        np.testing.assert_allclose(g["dbias"], bt.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("act", ["softmax", "gelu_tanh", "silu"])
def test_window_one_keeps_only_the_diagonal(act):
    """W = 1: query i sees key i alone, so softmax gives o_i = v_i and lse_i = s_ii, and GDPA
    gives o_i = act(s_ii) v_i (rows past the keys see nothing)."""
    pb = rand_problem(52, B=3, H=2, D=5, lq=[4, 6, 3], lk=[4, 5, 3], nb=3)
    scale = 0.6
    O, lse = run_oracle_fwd(pb, act, True, scale, 1)
    for b in range(3):
        for i in range(pb["qo"][b + 1] - pb["qo"][b]):
            q = pb["Q"][pb["qo"][b] + i]
            if i >= pb["ko"][b + 1] - pb["ko"][b]:
                np.testing.assert_array_equal(O[pb["qo"][b] + i], 0.0)
                continue
            k, v = pb["K"][pb["ko"][b] + i], pb["V"][pb["ko"][b] + i]
            s = scale * (q * k).sum(axis=1) + pb["bias"][:, 0]  # i - j = 0: bucket 0
            if act == "softmax":
                np.testing.assert_array_equal(O[pb["qo"][b] + i], v)
                np.testing.assert_allclose(lse[pb["qo"][b] + i], s, rtol=1e-14, atol=1e-14)
            else:
                a = oracle.act(act, s)
                np.testing.assert_allclose(O[pb["qo"][b] + i], a[:, None] * v, rtol=1e-13, atol=1e-14)


def test_window_covering_every_key_is_plain_causal():
    pb = rand_problem(53, B=4, H=2, D=3, maxlen=7, nb=4, same=False)
    for act in ("softmax", "silu"):
        O0, l0 = run_oracle_fwd(pb, act, True, 0.7)
        O1, l1 = run_oracle_fwd(pb, act, True, 0.7, 7)
        np.testing.assert_array_equal(O0, O1)
        np.testing.assert_array_equal(l0, l1)
        g0, g1 = run_oracle_bwd(pb, act, True, 0.7), run_oracle_bwd(pb, act, True, 0.7, 7)
        for k in ("dQ", "dK", "dV", "dbias"):
            np.testing.assert_array_equal(g0[k], g1[k])


def test_window_equals_attention_over_the_key_slice():
    """Without a bias, query i under window W is non-causal attention of that one query over keys
    max(0, i - W + 1) .. i: rebuild every query as its own sample with that key slice, and sum
    the slices' key gradients back (a different evaluation order of the same terms)."""
    W = 3
    pb = rand_problem(54, B=2, H=2, D=4, lq=[7, 5], lk=[7, 5])
    scale = 0.9
    for act in ("softmax", "gelu_tanh"):
        O, _ = run_oracle_fwd(pb, act, True, scale, W)
        g = run_oracle_bwd(pb, act, True, scale, W)
        qs, ks, rows = [], [], []
        for b in range(2):
            for i in range(pb["qo"][b + 1] - pb["qo"][b]):
                lo = max(0, i - W + 1)
                rows.append((pb["qo"][b] + i, pb["ko"][b] + lo, pb["ko"][b] + i + 1))
        qo = inputs.offsets_from_lengths(np.ones(len(rows), dtype=np.int64))
        ko = inputs.offsets_from_lengths(np.array([e - s for _, s, e in rows]))
        Qs = np.stack([pb["Q"][r] for r, _, _ in rows])
        dOs = np.stack([pb["dO"][r] for r, _, _ in rows])
        Ks = np.concatenate([pb["K"][s:e] for _, s, e in rows])
        Vs = np.concatenate([pb["V"][s:e] for _, s, e in rows])
        Os, _ = oracle.fwd(qo, ko, Qs, Ks, Vs, act=act, causal=False, scale=scale, nthreads=2)
        gs = oracle.bwd(qo, ko, Qs, Ks, Vs, dOs, act=act, causal=False, scale=scale, nthreads=2)
        idx = [r for r, _, _ in rows]
        np.testing.assert_allclose(O[idx], Os, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(g["dQ"][idx], gs["dQ"], rtol=1e-12, atol=1e-13)
        dK = np.zeros_like(pb["K"])
        dV = np.zeros_like(pb["V"])
        for n, (_, s, e) in enumerate(rows):
            dK[s:e] += gs["dK"][ko[n]:ko[n + 1]]
            dV[s:e] += gs["dV"][ko[n]:ko[n + 1]]
        np.testing.assert_allclose(g["dK"], dK, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g["dV"], dV, rtol=1e-12, atol=1e-13)


def test_window_bias_gradient_invariants():
    """Valid pairs have 0 <= i - j < W, so buckets W and above get nothing; softmax gradient
    rows sum to zero, so every head's buckets sum to zero."""
    W = 3
    pb = rand_problem(55, B=3, H=2, D=4, maxlen=9, nb=6, same=False)
    g = run_oracle_bwd(pb, "softmax", True, 0.7, W)
    np.testing.assert_array_equal(g["dbias"][:, W:], 0.0)
    np.testing.assert_allclose(g["dbias"].sum(axis=1), 0.0, atol=1e-12)
    assert np.abs(g["dbias"][:, :W]).min() > 0.0


# ----------------------------------------------------------------------------------------------
# activations


def test_activation_known_values():
    x = np.array([0.0])
    assert oracle.act("silu", x)[0] == 0.0
    assert oracle.act("gelu_tanh", x)[0] == 0.0
    assert abs(oracle.act("silu", x, derivative=True)[0] - 0.5) < 1e-15
    assert abs(oracle.act("gelu_tanh", x, derivative=True)[0] - 0.5) < 1e-15
    # large |x|: silu -> relu, gelu -> relu
    big = np.array([-30.0, 30.0])
    np.testing.assert_allclose(oracle.act("silu", big), [0.0, 30.0], atol=1e-11)
    np.testing.assert_allclose(oracle.act("gelu_tanh", big), [0.0, 30.0], atol=1e-11)


@pytest.mark.parametrize("name", ["silu", "gelu_tanh"])
def test_activation_vs_library_and_central_differences(name):
    x = np.linspace(-20, 20, 4001)
    t = torch.tensor(x, requires_grad=True)
    y = F.silu(t) if name == "silu" else F.gelu(t, approximate="tanh")
    y.sum().backward()
    np.testing.assert_allclose(oracle.act(name, x), y.detach().numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.act(name, x, derivative=True), t.grad.numpy(), rtol=1e-12,
                               atol=1e-14)
    h = 1e-6
    fd = (oracle.act(name, x + h) - oracle.act(name, x - h)) / (2 * h)
    assert np.abs(fd - oracle.act(name, x, derivative=True)).max() < 1e-8


# ----------------------------------------------------------------------------------------------
# MX decode


def _golden_mx():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_e8m0_spec_values.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, code, val = line.split()
            rows.append((kind, int(code, 16), float(val)))
    return rows


def test_mx_decode_spec_values():
    for kind, code, val in _golden_mx():
        dec = oracle.decode_e4m3 if kind == "e4m3" else oracle.decode_e8m0
        got = dec(np.array([code], np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(got), (kind, hex(code))
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (kind, hex(code))


def test_e4m3_decode_all_codes_against_library_dtype():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = oracle.decode_e4m3(codes)
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(ours)) and nan.sum() == 2
    assert np.array_equal(lib[~nan], ours[~nan])
    e8 = oracle.decode_e8m0(codes)
    assert np.isnan(e8[255]) and np.array_equal(e8[:255], np.ldexp(1.0, np.arange(255) - 127))


def test_mx_quantize_dequantize_roundtrip():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((257, 3, 64))
    codes, scales = inputs.mx_quantize(x)
    y = oracle.decode_mx(codes, scales)
    # elements that land in e4m3's normal range keep relative error <= 2^-4 (half an ulp);
    # blocks may saturate their largest element at 448 * scale (floor convention of the scale)
    sc = np.repeat(oracle.decode_e8m0(scales), 32, axis=-1)
    norm = (np.abs(x) / sc >= 2.0**-6) & (np.abs(x) / sc <= 448)
    rel = np.abs(y - x)[norm] / np.abs(x)[norm]
    assert rel.max() <= 2.0**-4
    # the encoder agrees with the library's own fp8 cast on the scaled values
    lib = torch.tensor(x / sc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inrange = np.abs(x / sc) <= 448
    assert np.array_equal(lib[inrange], codes[inrange])


# ----------------------------------------------------------------------------------------------
# counters


def test_pair_counter_brute_force():
    rng = np.random.default_rng(3)
    lq = rng.integers(0, 40, size=50)
    lk = rng.integers(0, 40, size=50)
    for causal in (False, True):
        got = workload.pairs_per_sample(lq, lk, causal)
        ref = [sum(1 for i in range(a) for j in range(b) if (not causal or j <= i))
               for a, b in zip(lq, lk)]
        assert list(got) == ref
    for W in (1, 2, 5, 17, 39, 100):
        got = workload.pairs_per_sample(lq, lk, True, W)
        ref = [sum(1 for i in range(a) for j in range(b) if i - W < j <= i) for a, b in zip(lq, lk)]
        assert list(got) == ref, W


def test_config_generators_shapes():
    p = inputs.config_problem(1)
    assert p.dtype == "f32" and p.B == 4 and p.H == 2 and p.D == 32
    assert np.array_equal(p.lq, p.lk) and p.lq.min() >= 1 and p.lq.max() <= 64
    p4 = inputs.config_problem(4, B=16)
    assert np.all(p4.lq == 32) and p4.lk.min() >= 16
    seeds = p4.Q.reshape(16, 32, 8, 64)
    assert np.all(seeds == seeds[:1])


# ---- block-aligned attention with rotary embeddings

def test_rope_closed_forms():
    """D = 2 turns (1, 0) to (cos p, sin p); position 0 is the identity; with D = 4 and base 100
    the second pair turns by p / 10."""
    p = np.array([0, 1, 2, 7])
    y = oracle.rope(np.tile(np.array([1.0, 0.0]), (4, 1, 1)), p)
    np.testing.assert_allclose(y[:, 0, 0], np.cos(p), atol=1e-15)
    np.testing.assert_allclose(y[:, 0, 1], np.sin(p), atol=1e-15)
    x = np.random.default_rng(80).standard_normal((3, 2, 8))
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(3, np.int64)), x)
    z = oracle.rope(np.array([[[0.0, 0.0, 0.0, 1.0]]]), np.array([3]), base=100.0)
    np.testing.assert_allclose(z[0, 0], [0.0, 0.0, -np.sin(0.3), np.cos(0.3)], atol=1e-15)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(81)
    q, k = rng.standard_normal((1, 1, 16)), rng.standard_normal((1, 1, 16))
    dot = lambda i, j: float((oracle.rope(q, np.array([i])) * oracle.rope(k, np.array([j]))).sum())
    for i, j in [(5, 2), (9, 9), (3, 11)]:
        for shift in (1, 17, 250):
            assert abs(dot(i, j) - dot(i + shift, j + shift)) < 1e-12
    assert abs(dot(0, 0) - float((q * k).sum())) < 1e-15


def test_rope_backward_is_the_transpose():
    rng = np.random.default_rng(82)
    x, g = rng.standard_normal((6, 2, 8)), rng.standard_normal((6, 2, 8))
    pos = np.array([0, 1, 5, 63, 64, 1000])
    lhs = float((oracle.rope(x, pos) * g).sum())
    rhs = float((x * oracle.rope_bwd(g, pos)).sum())
    assert abs(lhs - rhs) < 1e-12
    np.testing.assert_allclose(oracle.rope_bwd(oracle.rope(x, pos), pos), x, atol=1e-14)


def test_block_offsets():
    got = oracle.block_offsets(np.array([0, 130, 194, 194, 199]), 64)
    np.testing.assert_array_equal(np.diff(got), [64, 64, 2, 64, 5])


def _block_attention_loops(off, Q, K, V, act, causal, scale, block):
    """Pure-Python loops: rotate q_i and k_j at their positions in the sample (pairs (2m, 2m+1),
    angle p * 10000^(-2m/D)), then each query attends to the keys of its own block."""
    import math
    total, H, D = Q.shape
    O = np.zeros((total, H, D))

    def rot(v, p):
        out = [0.0] * D
        for m in range(D // 2):
            a = p * 10000.0 ** (-2.0 * m / D)
            out[2 * m] = math.cos(a) * v[2 * m] - math.sin(a) * v[2 * m + 1]
            out[2 * m + 1] = math.sin(a) * v[2 * m] + math.cos(a) * v[2 * m + 1]
        return out
    for b in range(len(off) - 1):
        s0, L = int(off[b]), int(off[b + 1] - off[b])
        for h in range(H):
            for i in range(L):
                qi = rot(Q[s0 + i, h], i)
                keys = [j for j in range(L) if j // block == i // block and (not causal or j <= i)]
                sc = []
                for j in keys:
                    kj = rot(K[s0 + j, h], j)
                    sc.append(scale * sum(qi[d] * kj[d] for d in range(D)))
                if act == "softmax":
                    mx = max(sc)
                    w = [math.exp(x - mx) for x in sc]
                    w = [x / sum(w) for x in w]
                else:  # silu
                    w = [x / (1.0 + math.exp(-x)) for x in sc]
                for wj, j in zip(w, keys):
                    O[s0 + i, h] += wj * V[s0 + j, h]
    return O


@pytest.mark.parametrize("act", ["softmax", "silu"])
@pytest.mark.parametrize("causal", [False, True])
def test_block_attention_brute_force_tiny(act, causal):
    rng = np.random.default_rng(83)
    off = np.array([0, 9, 12, 12, 17])
    Q, K, V = (rng.standard_normal((17, 2, 6)) for _ in range(3))
    got, _ = oracle.block_fwd(off, Q, K, V, act=act, causal=causal, scale=0.7, block=4)
    ref = _block_attention_loops(off, Q, K, V, act, causal, 0.7, 4)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_block_attention_short_samples_and_block_local_positions():
    """Samples no longer than a block are plain attention; rotary scores depend only on i - j, so
    rotating at block-local positions gives the same output as at sample positions."""
    rng = np.random.default_rng(84)
    off = np.array([0, 40, 104, 300])
    Q, K, V = (rng.standard_normal((300, 2, 16)) for _ in range(3))
    short = np.array([0, 40, 104])
    O1, _ = oracle.block_fwd(short, Q[:104], K[:104], V[:104], rotary=False)
    O2, _ = oracle.fwd(short, short, Q[:104], K[:104], V[:104])
    np.testing.assert_array_equal(O1, O2)
    bo = oracle.block_offsets(off, 64)
    bpos = oracle.local_positions(bo)
    O3, _ = oracle.fwd(bo, bo, oracle.rope(Q, bpos), oracle.rope(K, bpos), V, causal=True)
    O4, _ = oracle.block_fwd(off, Q, K, V, causal=True)
    np.testing.assert_allclose(O3, O4, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("act", ["softmax", "gelu_tanh"])
def test_block_attention_gradient_finite_differences(act):
    rng = np.random.default_rng(85)
    off = np.array([0, 7, 10])
    Q, K, V, dO = (rng.standard_normal((10, 1, 4)) for _ in range(4))
    kw = dict(act=act, causal=True, scale=0.9, block=4)
    g = oracle.block_bwd(off, Q, K, V, dO, **kw)

    def loss(q, k, v):
        O, _ = oracle.block_fwd(off, q, k, v, **kw)
        return float((O * dO).sum())
    h = 1e-6
    for name, key in (("Q", "dQ"), ("K", "dK"), ("V", "dV")):
        base = {"Q": Q, "K": K, "V": V}
        fd = np.zeros_like(base[name])
        for idx in np.ndindex(fd.shape):
            plus = {n: a.copy() for n, a in base.items()}
            minus = {n: a.copy() for n, a in base.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            fd[idx] = (loss(plus["Q"], plus["K"], plus["V"]) -
                       loss(minus["Q"], minus["K"], minus["V"])) / (2 * h)
        err = np.abs(fd - g[key]) / np.maximum(1.0, np.abs(g[key]))
        assert err.max() < 1e-6, (name, err.max())


def test_mx_quantize_threaded_chunks_give_the_same_bits():
    """Large arrays are quantised in row chunks by a thread pool; the bits equal one pass."""
    rng = np.random.default_rng(90)
    x = rng.standard_normal((70000, 2, 64), dtype=np.float32) * 3.0
    codes, scales = inputs.mx_quantize(x)
    c1, s1 = inputs._mx_quantize(x, 32)
    assert np.array_equal(codes, c1) and np.array_equal(scales, s1)


def test_config_generator_with_grad_keeps_input_bits():
    """Drawing dO for a forward-only workload leaves its Q, K, V (and MX scales) unchanged."""
    a = inputs.config_problem(5, B=3, seed=77)
    b = inputs.config_problem(5, B=3, seed=77, with_grad=True)
    for n in ("Q", "K", "V", "q_scale", "k_scale", "v_scale", "q_off", "kv_off"):
        assert np.array_equal(getattr(a, n), getattr(b, n)), n
    assert a.dO is None and b.dO.shape == (b.total_q, b.H, b.D)

"""Planted mistakes: the oracle's pins must reject a wrong oracle.

Each case copies the oracle's C source, changes one expression into a plausible mistake (a sign,
an index, a dropped factor, a wrong constant or bound), builds the altered copy on the CPU with
the same compiler line, runs a few of the pins of test_oracle.py against it, and requires that at
least one of them fails. The source in the repository is never modified; the GPU path is not
involved.
"""
import os

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdpa_oracle.c")


def _fwd_padded(act, causal, nb, same):
    return lambda: pins.test_fwd_matches_padded_library_attention(act, causal, nb, same, 0)


def _autograd(act, causal, nb, same):
    return lambda: pins.test_bwd_matches_torch_autograd(act, causal, nb, same)


# name: (expression in the source, its mistaken form, pins expected to notice)
PLANTS = {
    "softmax gradient sign": (
        "p[j] * (dp[j] - Di)", "p[j] * (dp[j] + Di)",
        [_autograd("softmax", True, 4, True), pins.test_softmax_backward_invariants]),
    "bias index transposed": (
        "if (nb > 0) v += bias_h[bias_index(i, j, nb)];",
        "if (nb > 0) v += bias_h[bias_index(j, i, nb)];",
        [_fwd_padded("softmax", True, 4, True), _fwd_padded("softmax", False, 5, False)]),
    "dQ scale dropped": (
        "dqi[c] += scale * ds[j] * kj[c];", "dqi[c] += ds[j] * kj[c];",
        [_autograd("gelu_tanh", False, 0, False),
         lambda: pins.test_bwd_finite_differences("softmax", True, 3)]),
    "dV weighted by the score gradient": (
        "dvj[c] += p[j] * doi[c];", "dvj[c] += ds[j] * doi[c];",
        [_autograd("silu", False, 3, False)]),
    "SiLU derivative sign": (
        "sg * (1.0 + x * (1.0 - sg))", "sg * (1.0 + x * (1.0 + sg))",
        [pins.test_activation_known_values,
         lambda: pins.test_activation_vs_library_and_central_differences("silu")]),
    "GELU cubic constant": (
        "static const double GELU_A = 0.044715;", "static const double GELU_A = 0.04472;",
        [lambda: pins.test_activation_vs_library_and_central_differences("gelu_tanh")]),
    "causal bound off by one": (
        "valid[j] = (unsigned char)((!causal || j <= i)",
        "valid[j] = (unsigned char)((!causal || j < i)",
        [_fwd_padded("softmax", True, 0, True), _fwd_padded("silu", True, 0, True)]),
    "window bound off by one": (
        "(window <= 0 || j > i - window)", "(window <= 0 || j >= i - window)",
        [lambda: pins.test_window_fwd_bwd_match_padded_library_attention("softmax", 3, 2),
         pins.test_window_bias_gradient_invariants]),
    "logsumexp in base 2": (
        "return m + log(l);", "return m + log2(l);",
        [pins.test_fwd_lse_against_library_logsumexp]),
    "e4m3 subnormal exponent": (
        "mag = ldexp((double)m / 8.0, -6);", "mag = ldexp((double)m / 8.0, -7);",
        [pins.test_mx_decode_spec_values, pins.test_e4m3_decode_all_codes_against_library_dtype]),
    "e8m0 exponent bias": (
        "return ldexp(1.0, (int)x - 127);", "return ldexp(1.0, (int)x - 128);",
        [pins.test_mx_decode_spec_values]),
    "error scale without the probability rounding term": (
        "wi += p[j] * p[j] * dp[j] * dp[j];", "wi += 0.0;",
        [lambda: pins.test_dbias_error_scale_monte_carlo(True),
         lambda: pins.test_dbias_error_scale_monte_carlo(False)]),
    "error scale without the output rounding term": (
        "wi += doi[c] * doi[c] * oc[c] * oc[c];", "wi += 0.0;",
        [lambda: pins.test_dbias_error_scale_monte_carlo(True),
         lambda: pins.test_dbias_error_scale_monte_carlo(False)]),
    "error scale with m in place of m squared": (
        "spart[r] += mr[r] * mr[r] * wi;", "spart[r] += mr[r] * wi;",
        [lambda: pins.test_dbias_error_scale_monte_carlo(True),
         lambda: pins.test_dbias_error_scale_monte_carlo(False)]),
}


@pytest.mark.parametrize("name", list(PLANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    expr, wrong, checks = PLANTS[name]
    src = open(SRC).read()
    assert src.count(expr) == 1, f"the expression to alter must occur once: {expr!r}"
    bad_src = tmp_path / "gdpa_oracle_planted.c"
    bad_src.write_text(src.replace(expr, wrong))
    lib = oracle.build(str(bad_src), str(tmp_path / "liboracle_planted.so"))
    caught = 0
    with oracle.using_library(lib):
        for check in checks:
            try:
                check()
            except Exception:  # an assertion, or the oracle rejecting its own output
                caught += 1
    assert caught > 0, f"no pin noticed the planted mistake: {name}"


def test_unaltered_copy_passes_the_same_pins(tmp_path):
    """The harness itself: a copy built the same way with no change passes every pin above."""
    lib = oracle.build(SRC, str(tmp_path / "liboracle_copy.so"))
    with oracle.using_library(lib):
        for _, _, checks in PLANTS.values():
            for check in checks:
                check()

"""Planted mistakes in a COPY of the oracle must each fail at least one pin.

Each mutation edits the C source text of the oracle (a dropped term, a wrong
sign, index or bound), builds it into a temporary library on the CPU and runs
every pin against it.  A mutation that no pin notices would mean the pins do
not fix that part of the oracle.
"""
import os

import pytest

import oracle
import oracle_pins

MUTATIONS = {
    "sink_dropped_from_denominator": (
        "double z = (sink[h] == -INFINITY) ? 0.0 : exp(sink[h] - m);", "double z = 0.0;"),
    "sink_counted_twice": (
        "double z = (sink[h] == -INFINITY) ? 0.0 : exp(sink[h] - m);",
        "double z = (sink[h] == -INFINITY) ? 0.0 : 2.0 * exp(sink[h] - m);"),
    "sink_scaled_like_a_logit": (
        "double z = (sink[h] == -INFINITY) ? 0.0 : exp(sink[h] - m);",
        "double z = (sink[h] == -INFINITY) ? 0.0 : exp(sink[h] * scale - m);"),
    "window_one_too_wide": ("dp < window", "dp <= window"),
    "causal_excludes_self": ("(dp >= 0)", "(dp > 0)"),
    "wrong_kv_group": ("const int g = h / group;", "const int g = h % hkv;"),
    "scale_missing": ("a[j] = dot * scale;", "a[j] = dot;"),
    "lse_without_max": ("m + log(z)", "log(z)"),
    "rope_sign_flipped": ("tmp[i1] = x0 * sin(phi) + x1 * cos(phi);",
                          "tmp[i1] = -x0 * sin(phi) + x1 * cos(phi);"),
    "rope_frequency_exponent": ("pow(base, -2.0 * (double)c / (double)rope_dim)",
                                "pow(base, -1.0 * (double)c / (double)rope_dim)"),
    "rope_pairs_swapped_style": ("const int i0 = style == 0 ? 2 * c : c;",
                                 "const int i0 = style == 1 ? 2 * c : c;"),
    "bf16_truncates": ("nearbyint(ldexp(a, -ulp_exp))", "floor(ldexp(a, -ulp_exp))"),
    "bwd_softmax_term_dropped": ("const double dA = s[j] * (dP - D);",
                                 "const double dA = s[j] * dP;"),
    "bwd_dsink_sign": ("dsink[h] -= p_sink * D;", "dsink[h] += p_sink * D;"),
    "bwd_dq_scale_missing": ("dqi[c] += scale * dA * kj[c];", "dqi[c] += dA * kj[c];"),
    "bwd_dv_weight_missing": ("dvj[c] += s[j] * di[c];", "dvj[c] += di[c];"),
    "bwd_D_without_output": ("D += di[c] * oi[c];", "D += di[c];"),
    "bwd_sink_share_unnormalised": ("exp(sink[h] - m) / z;", "exp(sink[h] - m);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, "mutation target not found: " + old
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = str(tmp_path / ("lib_%s.so" % name))
    oracle.build(force=True, src=str(mutated), out=so)
    lib = oracle.load_library(so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake " + name

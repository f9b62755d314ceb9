"""Plant plausible mistakes in copies of the oracle source and check that the
pins catch every one of them (CPU only; the real oracle is never modified).

Each mutant replaces exactly one snippet of gdn_oracle.c, is compiled into a
temporary library, and must fail at least one pin from oracle_pins.py.
"""
import os

import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    "conv taps reversed": ("w[(long)c * 4 + j] * x[src * D + c]",
                           "w[(long)c * 4 + (3 - j)] * x[src * D + c]"),
    "conv window shifted": ("long src = t - 3 + j;", "long src = t - 4 + j;"),
    "silu sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "l2 eps outside root": ("double inv = 1.0 / sqrt(ss + eps);\n        for (int c = 0; c < D; ++c)\n            out",
                            "double inv = 1.0 / (sqrt(ss) + eps);\n        for (int c = 0; c < D; ++c)\n            out"),
    "erase sign": ("S[(long)i * Dk + j] - b * Sk[i] * kt[j]", "S[(long)i * Dk + j] + b * Sk[i] * kt[j]"),
    "S transposed in S k": ("s += S[(long)i * Dk + j] * kt[j];", "s += S[(long)j * Dk + i] * kt[j];"),
    "decay on write term": ("a * erased + b * vt[i] * kt[j]", "a * (erased + b * vt[i] * kt[j])"),
    "beta dropped on write": ("a * erased + b * vt[i] * kt[j]", "a * erased + vt[i] * kt[j]"),
    "readout with k": ("s += S[(long)i * Dk + j] * qt[j];", "s += S[(long)i * Dk + j] * kt[j];"),
    "decay halved": ("double a = exp(log_a[t]), b = beta[t];",
                     "double a = exp(0.5 * log_a[t]), b = beta[t];"),
    "rms uses sum": ("1.0 / sqrt(ss / D + eps)", "1.0 / sqrt(ss + eps)"),
    "gate without silu": ("wc * silu(gate[t * D + c])", "wc * gate[t * D + c]"),
    "reverse not undone on store": ("y[(((long)b * T + SRC(t)) * H + h) * Dv + c] =",
                                    "y[(((long)b * T + t) * H + h) * Dv + c] ="),
    "conv weights of head 0": ("conv_k[((long)h * Dk + c) * 4 + j]", "conv_k[((long)c) * 4 + j]"),
    "S0 transposed": ("S0[((long)b * H + h) * Dv * Dk + i]",
                      "S0[((long)b * H + h) * Dv * Dk + (i % Dk) * Dv + i / Dk]"),
    "norm weight ignored": ("nw[c] = norm_w ? norm_w[(long)h * Dv + c] : 1.0;", "nw[c] = 1.0;"),
    "q not normalised": ("oracle_l2_normalize(T, Dk, tmp, eps_l2, qh);",
                         "memcpy(qh, tmp, sizeof(double) * (size_t)T * Dk);"),
    "state after readout": (
        "        for (int i = 0; i < Dv; ++i) {\n            double s = 0.0;\n            for (int j = 0; j < Dk; ++j)\n                s += S[(long)i * Dk + j] * qt[j];\n            o[t * Dv + i] = s;\n        }\n",
        ""),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"snippet for '{name}' must occur exactly once"
    mutated = source.replace(old, new)
    if name == "state after readout":
        # move the readout in front of the state update instead of dropping it
        anchor = "        for (int i = 0; i < Dv; ++i) {\n            double s = 0.0;\n            for (int j = 0; j < Dk; ++j)\n                s += S[(long)i * Dk + j] * kt[j];"
        assert mutated.count(anchor) == 1
        mutated = mutated.replace(anchor, MUTANTS[name][0] + anchor)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib = oracle.compile_source(str(src), str(tmp_path / f"libmutant_{abs(hash(name))}.so"))
    o = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant '{name}' passed every pin"
    os.remove(lib)

"""The seeded input generator (CPU)."""
import numpy as np
import torch

import gdn_inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 5, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(gdn_inputs.round_bf16(x), ref)


def test_generator_is_seeded_and_shaped():
    a = gdn_inputs.generate(1, T=300)
    b = gdn_inputs.generate(1, T=300)
    for key in a:
        if a[key] is None:
            assert b[key] is None
        else:
            assert np.array_equal(a[key], b[key]), key
    assert a["q"].shape == (1, 300, 12, 128)
    assert np.array_equal(gdn_inputs.round_bf16(a["q"]), a["q"])
    assert a["log_a"].shape == (1, 300, 12) and np.all(a["log_a"] <= 0)
    assert np.all((a["beta"] > 0) & (a["beta"] < 1))
    assert a["S0"] is None and gdn_inputs.generate(3, T=10)["S0"].shape == (1, 24, 128, 128)


def test_distributions():
    d = gdn_inputs.generate(0)
    assert abs(d["q"].std() - 1) < 0.02 and abs(d["conv_q"].std() - 0.5) < 0.05
    # log a = -r_h softplus(x), r_h in [0.01, 0.1], x ~ N(0,1): the median of
    # softplus(x) is ln 2, so each head's median -log a lies in [0.01, 0.1] ln 2
    med = np.median(-d["log_a"], axis=(0, 1))
    assert np.all((med > 0.0095 * np.log(2)) & (med < 0.105 * np.log(2)))

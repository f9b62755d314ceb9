"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: relative L2 error <= 1e-2 with bf16 I/O and <= 1e-4 with fp32 I/O, on
the output y and on the final state(s); in addition every single token-head
of y must be within 5x the bar.
"""
import numpy as np
import pytest
import torch

import gdn_inputs
import oracle
from tests.gpu_common import check, compare_workload, run_gpu, say

pytestmark = pytest.mark.gpu

W = gdn_inputs.WORKLOADS


@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_reduced_workload(wid):
    """Each workload's distributions at T = 5 chunks + a 37-token tail, 2 heads."""
    w = W[wid]
    compare_workload(w, T=64 * 5 + 37, H=2)


@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_full_workload(wid):
    """Each workload at its full size, all heads compared."""
    compare_workload(W[wid])


def test_cfg_pair_batch():
    """A classifier-free-guidance pair as one call: B = 2 at the full
    480x832 length (T = 32760, H = 12, d = 128), every head of both rows."""
    compare_workload(W[1], B=2, seed=4242)


@pytest.mark.parametrize("wid", [0, 1])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 63, 64, 65, 129])
def test_edge_lengths(wid, T):
    """Short sequences (inside the conv window, one chunk, chunk boundaries),
    two batch rows, three heads, a random initial state."""
    w = W[wid]
    inp = gdn_inputs.generate(w, T=T, H=3, B=2, seed=77 + T)
    inp["S0"] = (0.05 * np.random.default_rng(T).standard_normal((2, 3, w.D, w.D))).astype(np.float32)
    inp["norm_w"] = (1 + 0.3 * np.random.default_rng(5).standard_normal((3, w.D))).astype(np.float32)
    say(f"case: edge T={T} workload {wid}")
    y, s = run_gpu(inp, w.dtype)
    ry, rs, _ = oracle.inputs_for(inp)
    check("y", y, ry, w.dtype)
    check("S_T", s, rs, w.dtype)


def test_bf16_d64():
    w = gdn_inputs.Workload(90, "bf16 d64", 1, 1000, 4, 64, "bf16")
    compare_workload(w)


@pytest.mark.parametrize("wid", [0, 1])
def test_reverse_scan(wid):
    compare_workload(W[wid], T=64 * 3 + 5, H=2, reverse=True)


def test_deterministic():
    inp = gdn_inputs.generate(1, T=1000, H=3)
    y1, s1 = run_gpu(inp, "bf16")
    y2, s2 = run_gpu(inp, "bf16")
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_closed_form_pure_decay():
    """b = 0: S_t = (prod a) S0, so S_T is S0 scaled by the total decay and y is
    the normalised decayed readout; checked on the GPU path."""
    w = W[1]
    inp = gdn_inputs.generate(w, T=300, H=2, seed=5)
    inp["beta"][:] = 0.0
    S0 = (0.1 * np.random.default_rng(3).standard_normal((1, 2, 128, 128))).astype(np.float32)
    inp["S0"] = S0
    y, s = run_gpu(inp, "bf16")
    decay = np.exp(np.sum(inp["log_a"][0].astype(np.float64), axis=0))  # [H]
    np.testing.assert_allclose(s[0], decay[:, None, None] * S0[0], rtol=2e-3, atol=1e-7)
    ry, _, _ = oracle.inputs_for(inp)
    check("y", y, ry, "bf16")


def test_closed_form_exact_retrieval():
    """a = 1, b = 1, identity conv taps and one-hot keys: the state is a lookup
    table, S_T e_i = v^ of the last token whose key is e_i."""
    D, T, H = 64, 96, 1
    rng = np.random.default_rng(9)
    keys = np.concatenate([rng.permutation(D), rng.permutation(D)[:32]])
    inp = dict(
        q=np.eye(D, dtype=np.float32)[rng.integers(0, D, T)][None, :, None] * 2.0,
        k=np.eye(D, dtype=np.float32)[keys][None, :, None] * 2.0,
        v=rng.standard_normal((1, T, H, D)).astype(np.float32),
        gate=rng.standard_normal((1, T, H, D)).astype(np.float32),
        log_a=np.zeros((1, T, H), np.float32), beta=np.ones((1, T, H), np.float32),
        conv_q=np.tile(np.array([0, 0, 0, 1], np.float32), (D, 1)),
        conv_k=np.tile(np.array([0, 0, 0, 1], np.float32), (D, 1)),
        conv_v=np.tile(np.array([0, 0, 0, 1], np.float32), (D, 1)),
        norm_w=np.ones((1, D), np.float32), S0=None)
    _, s = run_gpu(inp, "f32")
    vhat = inp["v"][0, :, 0].astype(np.float64)
    vhat = vhat / (1 + np.exp(-vhat))
    for col in range(D):
        last = max(t for t in range(T) if keys[t] == col)
        np.testing.assert_allclose(s[0, 0, :, col], vhat[last], rtol=1e-4, atol=1e-5)


def test_errors_leave_outputs_untouched():
    import linear_attention_token_fwd_amd as gdn
    inp = gdn_inputs.generate(1, T=100, H=2)
    d = gdn.to_device(inp, dtype=torch.bfloat16)
    out = torch.full((1, 100, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_fwd(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["gate"], d["conv_q"],
                    d["conv_k"], d["conv_v"], out=out, workspace=small)
    assert e.value.status == gdn.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

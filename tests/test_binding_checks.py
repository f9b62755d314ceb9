"""Checks the Python binding makes before anything reaches the C layer (CPU).

The C entry points cannot see tensor sizes, so the binding checks what only
it can: that a variable-length batch's offset table starts at 0, increases,
and ends at the packed row count of the tensors, and that every tensor of
the backward of a variable-length batch has the dtype and shape the C layer
will read.  These run on host tensors: every mismatch must raise before the
device check (and long before a launch).
"""
import pytest
import torch

import linear_attention_token_fwd_amd as gdn

H, D = 2, 64


def _fwd_args(total, dtype=torch.float32):
    q = torch.zeros((1, total, H, D), dtype=dtype)
    g = torch.zeros((1, total, H))
    w = torch.zeros((H * D, 4))
    return q, q.clone(), q.clone(), g, g.clone(), q.clone(), w, w.clone(), w.clone()


BAD_TABLES = [
    ([1, 10], "start at 0"),
    ([0, 5, 5, 10], "increase"),
    ([0, 6, 4, 10], "increase"),
    ([0, 4, 12], "ends at 12"),
    ([0, 4, 8], "ends at 8"),
    ([0], "at least two"),
]


@pytest.mark.parametrize("table,msg", BAD_TABLES)
def test_fwd_varlen_table_checked_against_tensors(table, msg):
    with pytest.raises(ValueError, match=msg):
        gdn.gdn_fwd_varlen(*_fwd_args(10), table)


@pytest.mark.parametrize("table,msg", BAD_TABLES)
def test_bwd_varlen_table_checked_against_tensors(table, msg):
    q, k, v, la, b, gate, cq, ck, cv = _fwd_args(10)
    with pytest.raises(ValueError, match=msg):
        gdn.gdn_bwd_varlen(q, k, v, la, b, gate, cq, ck, cv, None, None, q.clone(), None, table)


def _bwd_case(**override):
    q, k, v, la, b, gate, cq, ck, cv = _fwd_args(10)
    args = dict(q=q, k=k, v=v, log_a=la, beta=b, gate=gate, conv_q=cq, conv_k=ck, conv_v=cv,
                norm_w=torch.ones((H, D)), S0=torch.zeros((2, H, D, D)), dy=q.clone(),
                dS_T=torch.zeros((2, H, D, D)))
    args.update(override)
    return args


BWD_MISMATCHES = [
    ("log_a", torch.zeros((1, 10, H), dtype=torch.bfloat16), TypeError),
    ("beta", torch.zeros((1, 9, H)), ValueError),
    ("k", torch.zeros((1, 10, H, D), dtype=torch.bfloat16), TypeError),
    ("v", torch.zeros((1, 10, H, D + 1)), ValueError),
    ("gate", torch.zeros((1, 10, H + 1, D)), ValueError),
    ("dy", torch.zeros((1, 11, H, D)), ValueError),
    ("conv_k", torch.zeros((H * D, 3)), ValueError),
    ("norm_w", torch.zeros((H, D), dtype=torch.float64), TypeError),
    ("S0", torch.zeros((3, H, D, D)), ValueError),
    ("dS_T", torch.zeros((2, H, D, D), dtype=torch.bfloat16), TypeError),
    ("q", torch.zeros((1, 10, H, 2 * D))[..., ::2], ValueError),
]


@pytest.mark.parametrize("name,bad,exc", BWD_MISMATCHES, ids=[m[0] for m in BWD_MISMATCHES])
def test_bwd_varlen_checks_every_tensor(name, bad, exc):
    a = _bwd_case(**{name: bad})
    if name == "q":  # a strided view of the right shape
        a["q"] = bad
    with pytest.raises(exc):
        gdn.gdn_bwd_varlen(a["q"], a["k"], a["v"], a["log_a"], a["beta"], a["gate"], a["conv_q"], a["conv_k"],
                           a["conv_v"], a["norm_w"], a["S0"], a["dy"], a["dS_T"], [0, 4, 10])


def test_bwd_varlen_host_tensors_refused_after_checks():
    a = _bwd_case()
    with pytest.raises(TypeError, match="device tensor"):
        gdn.gdn_bwd_varlen(a["q"], a["k"], a["v"], a["log_a"], a["beta"], a["gate"], a["conv_q"], a["conv_k"],
                           a["conv_v"], a["norm_w"], a["S0"], a["dy"], a["dS_T"], [0, 4, 10])

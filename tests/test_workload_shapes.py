"""The workload shapes against the one table on the pages that prints numbers
for the Wan2.1-1.3B model (T3-Video page, Table 1).

With 30 blocks, hidden width H*D and T latent tokens, a DiT forward spends
  QKV projection: 30 * T * 3 * (H*D)^2 MACs,
  O projection:   30 * T * (H*D)^2 MACs,
  softmax attention (Q K^T and A V): 30 * 2 * T^2 * (H*D) MACs.
The table's printed values must come out of the 480x832 and 720x1280
workloads' T, H and D to the table's printed precision.
"""
import json
import os

import gdn_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_table1_macs_match_workload_shapes():
    with open(os.path.join(HERE, "golden", "t3video_table1_wan21_macs.json")) as f:
        g = json.load(f)
    tol = g["printed_precision"] / 2 + 1e-6 * 1e12
    for key, wid in (("480x832", 1), ("720x1280", 2)):
        w = gdn_inputs.WORKLOADS[wid]
        hidden = w.H * w.D
        row = g["rows"][key]
        L = g["blocks"]
        assert abs(L * w.T * 3 * hidden ** 2 - row["qkv_proj"]) <= tol
        assert abs(L * w.T * hidden ** 2 - row["o_proj"]) <= tol
        assert abs(L * 2 * w.T ** 2 * hidden - row["attn"]) <= tol


def test_latent_grids():
    # frames -> latent frames (1 + (F-1)/4), pixels -> 16x16 patches
    grid = {1: (81, 480, 832), 2: (81, 720, 1280), 4: (321, 480, 832)}
    for wid, (F, Hp, Wp) in grid.items():
        w = gdn_inputs.WORKLOADS[wid]
        assert w.T == (1 + (F - 1) // 4) * (Hp // 16) * (Wp // 16)
    assert gdn_inputs.WORKLOADS[3].T == 31 * 22 * 40

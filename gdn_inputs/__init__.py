"""Seeded synthetic inputs for the GDN layer forward.

This module is shared by the tests, the benchmark and the smoke check.  It
holds the workload shapes and the random draws only: none of the layer's
arithmetic lives here, and it imports neither the oracle nor the HIP binding.

The shapes stand in for Wan2.1 video latents.  The T3-Video page (Table 1,
Wan2.1-T2V-1.3B parameters and MACs) fixes the 1.3B model's attention width at
1536 = 12 heads x 128 and its token counts: 21x30x52 = 32760 latent tokens at
480x832 and 21x45x80 = 75600 at 720x1280 (81 frames).  The LinMorph page
("Acceleration grows with video length") measures 321 frames at 480x832,
i.e. 81x30x52 = 126360 tokens.  No dataset is involved: every tensor is drawn
from a fixed distribution with a fixed seed.

Draw order per workload (numpy PCG64, seed 1000 + workload id):
  q, k, v, gate ~ N(0, 1) elementwise, [B, T, H, D], drawn as float32;
  conv_q, conv_k, conv_v ~ N(0, 0.5^2) (0.5 is the standard deviation), [H*D, 4];
  z ~ N(0, 1) [B, T, H]   -> beta = sigmoid(z);
  x ~ N(0, 1) [B, T, H]   -> log_a = -exp(A_h) * softplus(x);
  A_h ~ U(ln 0.01, ln 0.1) per head;
  S0 ~ N(0, 0.02^2) [B, H, Dv, Dk] for the workload with an initial state.
For bf16 workloads q, k, v and gate are rounded to bf16 (round to nearest
even) and carried as float32 arrays holding the rounded values.

Token mixer projections (generate_mixer, seed 2000 + id unless given), model
width C, in this order:
  x ~ N(0, 1) [B, T, C]                      (hidden states, bf16);
  w_in ~ N(0, 1/C) [4*H*D + 2*H, C]          (bf16; unit-variance outputs);
  b_in ~ N(0, 0.1^2) [4*H*D + 2*H]           (fp32);
  A_log ~ U(ln 0.01, ln 0.1) [H];
  w_out ~ N(0, 1/(H*D)) [C, H*D]             (bf16);
  b_out ~ N(0, 0.1^2) [C];
  conv_q, conv_k, conv_v ~ N(0, 0.5^2) [H*D, 4]; norm_w = 1.
The 1.3B model's width is C = 1536 = 12 x 128 (T3-Video page, Table 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    B: int
    T: int
    H: int
    D: int
    dtype: str          # "f32" or "bf16": dtype of q, k, v, gate and y
    has_S0: bool = False
    bidirectional: bool = False
    chunk: int = 64

    @property
    def tokens(self) -> int:
        return self.B * self.T


@dataclass(frozen=True)
class MixerWorkload:
    id: int
    name: str
    B: int
    T: int
    H: int
    D: int
    C: int

    @property
    def tokens(self) -> int:
        return self.B * self.T


MIXER_WORKLOADS = [
    MixerWorkload(0, "small mixer: B1 T700 H3 d64 C192", 1, 700, 3, 64, 192),
    MixerWorkload(1, "Wan2.1-1.3B token mixer, 480x832, 81 frames: B1 T32760 H12 d128 C1536",
                  1, 32760, 12, 128, 1536),
]


WORKLOADS = [
    Workload(0, "tiny fp32: B1 H2 T2048 d64", 1, 2048, 2, 64, "f32"),
    Workload(1, "Wan2.1-1.3B layer, 480x832, 81 frames (21x30x52): B1 H12 T32760 d128 bf16",
             1, 32760, 12, 128, "bf16"),
    Workload(2, "720x1280, 81 frames (21x45x80): B1 H12 T75600 d128 bf16",
             1, 75600, 12, 128, "bf16"),
    Workload(3, "wide model (31x22x40): B1 H24 T27280 d128 bf16, random initial state",
             1, 27280, 24, 128, "bf16", has_S0=True),
    Workload(4, "321 frames at 480x832 (81x30x52): B1 H12 T126360 d128 bf16, bidirectional",
             1, 126360, 12, 128, "bf16", bidirectional=True),
]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns
    float32 holding the rounded values.  NaN/Inf are not expected here."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = u + np.uint32(0x7FFF)
    r += lsb
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _softplus(x):
    return np.where(x > 20.0, x, np.log1p(np.exp(np.minimum(x, 20.0))))


def generate(w: Workload | int, seed: int | None = None, T: int | None = None,
             H: int | None = None, B: int | None = None) -> dict:
    """Draw one workload's inputs.

    T/H/B override the workload's sizes (for reduced parity cases); the
    distributions stay those of the workload.  Returns a dict of float32
    numpy arrays: q, k, v, gate [B,T,H,D]; log_a, beta [B,T,H];
    conv_q, conv_k, conv_v [H*D, 4]; norm_w [H, D] (ones); S0 or None.
    """
    if isinstance(w, int):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    D = w.D
    rng = np.random.default_rng(1000 + w.id if seed is None else seed)
    shp = (B, T, H, D)
    q = rng.standard_normal(shp, dtype=np.float32)
    k = rng.standard_normal(shp, dtype=np.float32)
    v = rng.standard_normal(shp, dtype=np.float32)
    gate = rng.standard_normal(shp, dtype=np.float32)
    conv_q = (0.5 * rng.standard_normal((H * D, 4))).astype(np.float32)
    conv_k = (0.5 * rng.standard_normal((H * D, 4))).astype(np.float32)
    conv_v = (0.5 * rng.standard_normal((H * D, 4))).astype(np.float32)
    z = rng.standard_normal((B, T, H))
    x = rng.standard_normal((B, T, H))
    A_h = rng.uniform(np.log(0.01), np.log(0.1), size=H)
    beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    log_a = (-np.exp(A_h)[None, None, :] * _softplus(x)).astype(np.float32)
    S0 = None
    if w.has_S0:
        S0 = (0.02 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    if w.dtype == "bf16":
        q, k, v, gate = (round_bf16(a) for a in (q, k, v, gate))
    norm_w = np.ones((H, D), np.float32)
    return dict(q=q, k=k, v=v, gate=gate, log_a=log_a, beta=beta, conv_q=conv_q,
                conv_k=conv_k, conv_v=conv_v, norm_w=norm_w, S0=S0)


def generate_grads(w: Workload | int, seed: int, T: int | None = None, H: int | None = None,
                   B: int | None = None, t_end: int | None = None, state: bool = True) -> dict:
    """Draw the upstream gradients of a backward pass (seed as given): dy ~
    N(0, 1) [B, T, H, D] (rounded to bf16 for bf16 workloads), zero from
    token t_end on if t_end is given; dS_T ~ N(0, 1) [B, H, D, D], or None
    if not state.  float32 numpy arrays."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((B, T, H, w.D), dtype=np.float32)
    if t_end is not None:
        dy[:, t_end:] = 0.0
    if w.dtype == "bf16":
        dy = round_bf16(dy)
    dS_T = rng.standard_normal((B, H, w.D, w.D), dtype=np.float32) if state else None
    return dict(dy=dy, dS_T=dS_T)


def generate_mixer(w: MixerWorkload | int, seed: int | None = None, T: int | None = None,
                   B: int | None = None, bias: bool = True) -> dict:
    """Draw a token mixer's hidden states and weights (float32 numpy arrays
    holding bf16 values where the device tensor is bf16): x, w_in, b_in,
    A_log, w_out, b_out, conv_q, conv_k, conv_v, norm_w.  bias=False gives
    b_in = b_out = None (the same draws otherwise)."""
    if isinstance(w, int):
        w = MIXER_WORKLOADS[w]
    B = w.B if B is None else B
    T = w.T if T is None else T
    H, D, C = w.H, w.D, w.C
    HD, N = H * D, 4 * H * D + 2 * H
    rng = np.random.default_rng(2000 + w.id if seed is None else seed)
    x = round_bf16(rng.standard_normal((B, T, C), dtype=np.float32))
    w_in = round_bf16(rng.standard_normal((N, C), dtype=np.float32) / np.float32(np.sqrt(C)))
    b_in = (0.1 * rng.standard_normal(N)).astype(np.float32)
    A_log = rng.uniform(np.log(0.01), np.log(0.1), size=H).astype(np.float32)
    w_out = round_bf16(rng.standard_normal((C, HD), dtype=np.float32) / np.float32(np.sqrt(HD)))
    b_out = (0.1 * rng.standard_normal(C)).astype(np.float32)
    conv = [(0.5 * rng.standard_normal((HD, 4))).astype(np.float32) for _ in range(3)]
    return dict(x=x, w_in=w_in, b_in=b_in if bias else None, A_log=A_log, w_out=w_out,
                b_out=b_out if bias else None, conv_q=conv[0], conv_k=conv[1], conv_v=conv[2],
                norm_w=np.ones((H, D), np.float32))

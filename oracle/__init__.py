"""fp64 CPU oracle of one Gated DeltaNet (GDN) layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and never imports it.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, one function per part
of the layer: short convolution + SiLU, L2 normalisation, the gated delta rule
token by token, gated RMS normalisation).  This module only builds that file,
marshals numpy arrays and, for the bidirectional variant, adds the two scans.
``chunked.py`` holds an independent fp64 model of the chunked (WY) form used to
pin the sequential recurrence by brute force.

Sources: LinMorph project page ("Abstract", "Why learn the initialization?":
the GDN module and its parameter groups); VMonarch page, section 2 "Efficient
Attention Mechanisms" and ref. [57] (GDN as a linear-attention mixer with an
expanded recurrent state).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gdn_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int)


def compile_source(src: str, out: str) -> str:
    """gcc a C oracle source into a shared library (generic x86-64, OpenMP)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(LIB_PATH):
        compile_source(SOURCE, LIB_PATH)
    return LIB_PATH


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


def _f(a):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_fp)


class Oracle:
    """The oracle's functions bound to one compiled library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        lib.oracle_short_conv_silu.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _dp, _dp]
        lib.oracle_short_conv_silu.restype = None
        lib.oracle_l2_normalize.argtypes = [ctypes.c_long, ctypes.c_int, _dp, ctypes.c_double, _dp]
        lib.oracle_l2_normalize.restype = None
        lib.oracle_delta_rule.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                          _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.oracle_delta_rule.restype = None
        lib.oracle_gated_rmsnorm.argtypes = [ctypes.c_long, ctypes.c_int, _dp, _dp, _dp,
                                             ctypes.c_double, _dp]
        lib.oracle_gated_rmsnorm.restype = None
        lib.oracle_gdn_fwd.argtypes = [
            ctypes.c_int, ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            _fp, _fp, _fp, _fp, _fp, _fp, _fp, _fp, _fp, _fp,
            ctypes.c_double, ctypes.c_double, _fp, ctypes.c_int, _dp, _dp,
            _ip, ctypes.c_int, ctypes.c_int]
        lib.oracle_gdn_fwd.restype = ctypes.c_int
        self.lib = lib

    # ------------------------------------------------------------ the parts
    def short_conv_silu(self, x, w):
        """x [T, D], w [D, 4] -> SiLU(causal depthwise 4-tap conv), fp64 [T, D]."""
        x, xp = _d(x)
        w, wp = _d(w)
        T, D = x.shape
        assert w.shape == (D, 4)
        out = np.empty((T, D), np.float64)
        self.lib.oracle_short_conv_silu(T, D, xp, wp, out.ctypes.data_as(_dp))
        return out

    def l2_normalize(self, x, eps=1e-6):
        x, xp = _d(x)
        T, D = x.shape
        out = np.empty((T, D), np.float64)
        self.lib.oracle_l2_normalize(T, D, xp, eps, out.ctypes.data_as(_dp))
        return out

    def delta_rule(self, q, k, v, log_a, beta, S0=None, return_states=False):
        """Token-by-token gated delta rule on one head.

        q, k [T, Dk]; v [T, Dv]; log_a, beta [T]; S0 [Dv, Dk] or None.
        Returns (o [T, Dv], S_T [Dv, Dk]) and, if return_states, also the
        state after every token [T, Dv, Dk].
        """
        q, qp = _d(q)
        k, kp = _d(k)
        v, vp = _d(v)
        _la, lap = _d(np.asarray(log_a).reshape(-1))
        _be, bep = _d(np.asarray(beta).reshape(-1))
        T, Dk = q.shape
        Dv = v.shape[1]
        S = (np.zeros((Dv, Dk), np.float64) if S0 is None
             else np.array(S0, np.float64, copy=True, order="C"))
        o = np.empty((T, Dv), np.float64)
        hist = np.empty((T, Dv, Dk), np.float64) if return_states else None
        self.lib.oracle_delta_rule(T, Dk, Dv, qp, kp, vp, lap, bep, S.ctypes.data_as(_dp),
                                   o.ctypes.data_as(_dp),
                                   hist.ctypes.data_as(_dp) if return_states else None)
        if return_states:
            return o, S, hist
        return o, S

    def gated_rmsnorm(self, o, gate, w=None, eps=1e-6):
        o, op = _d(o)
        _g, gp = _d(gate)
        T, D = o.shape
        wp = None
        if w is not None:
            w, wp = _d(w)
        y = np.empty((T, D), np.float64)
        self.lib.oracle_gated_rmsnorm(T, D, op, gp, wp, eps, y.ctypes.data_as(_dp))
        return y

    # ------------------------------------------------------------ the layer
    def gdn_fwd(self, q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w=None,
                S0=None, eps_l2=1e-6, eps_norm=1e-6, reverse=False, heads=None, threads=0):
        """Whole layer in fp64.

        Array arguments hold the exact values the GPU receives (bf16 or fp32
        values, widened to float32 without rounding).  Shapes: q, k
        [B,T,H,Dk]; v, gate [B,T,H,Dv]; log_a, beta [B,T,H]; conv_* [H*D, 4];
        norm_w [H, Dv] or None; S0 [B,H,Dv,Dk] or None.  heads: optional head
        subset (y of other heads is NaN).
        Returns (y [B,T,H,Dv] fp64, S_T [B,H,Dv,Dk] fp64, threads_used).
        """
        B, T, H, Dk = q.shape
        Dv = v.shape[3]
        arrs = [_f(a) for a in (q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v,
                                norm_w, S0)]
        keep = [a for a, _ in arrs]  # keep the contiguous copies alive
        ptrs = [p for _, p in arrs]
        y = np.full((B, T, H, Dv), np.nan, np.float64)
        S_T = np.full((B, H, Dv, Dk), np.nan, np.float64)
        if heads is None:
            hp, nh = None, H
        else:
            harr = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
            keep.append(harr)
            hp, nh = harr.ctypes.data_as(_ip), len(harr)
        used = self.lib.oracle_gdn_fwd(B, T, H, Dk, Dv, *ptrs[:10], eps_l2, eps_norm,
                                       ptrs[10], 1 if reverse else 0,
                                       y.ctypes.data_as(_dp), S_T.ctypes.data_as(_dp),
                                       hp, nh, int(threads))
        del keep
        if used < 0:
            raise MemoryError("oracle_gdn_fwd: allocation failed")
        return y, S_T, used

    def gdn_fwd_bidir(self, q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v,
                      norm_w=None, S0=None, eps_l2=1e-6, eps_norm=1e-6, heads=None,
                      threads=0):
        """Bidirectional stress variant: the whole layer run once forward in
        time and once on the time-reversed sequence (each scan with its own
        causal convolution and output normalisation); outputs added in fp64.

        Returns (y, S_T_forward, S_T_reversed, threads_used).
        """
        yf, sf, used = self.gdn_fwd(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v,
                                    norm_w, S0, eps_l2, eps_norm, False, heads, threads)
        yr, sr, _ = self.gdn_fwd(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v,
                                 norm_w, S0, eps_l2, eps_norm, True, heads, threads)
        return yf + yr, sf, sr, used


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from gdn_oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _default = Oracle(LIB_PATH)
    return _default


def short_conv_silu(*a, **kw):
    return get().short_conv_silu(*a, **kw)


def l2_normalize(*a, **kw):
    return get().l2_normalize(*a, **kw)


def delta_rule(*a, **kw):
    return get().delta_rule(*a, **kw)


def gated_rmsnorm(*a, **kw):
    return get().gated_rmsnorm(*a, **kw)


def gdn_fwd(*a, **kw):
    return get().gdn_fwd(*a, **kw)


def gdn_fwd_bidir(*a, **kw):
    return get().gdn_fwd_bidir(*a, **kw)


def inputs_for(inp: dict, reverse=False, heads=None, threads=0, bidir=False):
    """Run the layer on a dict produced by the seeded input generator."""
    args = (inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], inp["gate"],
            inp["conv_q"], inp["conv_k"], inp["conv_v"], inp.get("norm_w"), inp.get("S0"))
    if bidir:
        return gdn_fwd_bidir(*args, heads=heads, threads=threads)
    return gdn_fwd(*args, reverse=reverse, heads=heads, threads=threads)

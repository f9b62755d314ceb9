"""Python binding of libgdn.so, the gfx950 Gated DeltaNet layer forward.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI of ``include/gdn.h``; torch supplies device memory and the
stream.  The names match the C entry points.  If the library has not been
built (``python -m linear_attention_token_fwd_amd.build``) every entry point
raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, or another build of the same sources named by GDN_LIBRARY
# (the host-sanitizer test loads an instrumented build this way)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_ALIGNMENT, GDN_ERR_WORKSPACE, GDN_ERR_HIP = range(6)
GDN_F32, GDN_BF16 = 0, 1

EXPORTS = ("gdn_fwd", "gdn_fwd_bidir", "gdn_fwd_workspace_bytes", "gdn_fwd_bidir_workspace_bytes",
           "gdn_fwd_launch_count", "gdn_fwd_launch_name", "gdn_fwd_timed", "gdn_status_string",
           "gdn_in_proj", "gdn_out_proj", "gdn_mixer_workspace_bytes", "gdn_mixer_fwd", "gdn_mixer_fwd_timed",
           "gdn_fwd_varlen", "gdn_fwd_varlen_workspace_bytes", "gdn_set_graph_cache_limit",
           "gdn_graph_cache_count", "gdn_bwd", "gdn_bwd_workspace_bytes", "gdn_bwd_timed",
           "gdn_bwd_launch_count", "gdn_bwd_launch_name", "gdn_bwd_varlen", "gdn_bwd_varlen_workspace_bytes",
           "gdn_fwd_noalloc")


class GdnFwdParams(ctypes.Structure):
    """Mirror of ``gdn_fwd_params`` in include/gdn.h."""
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
        ("Dk", ctypes.c_int), ("Dv", ctypes.c_int), ("io_dtype", ctypes.c_int),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("log_a", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("gate", ctypes.c_void_p),
        ("conv_q", ctypes.c_void_p), ("conv_k", ctypes.c_void_p), ("conv_v", ctypes.c_void_p),
        ("norm_w", ctypes.c_void_p), ("eps_l2", ctypes.c_float), ("eps_norm", ctypes.c_float),
        ("S0", ctypes.c_void_p), ("o", ctypes.c_void_p), ("S_T", ctypes.c_void_p),
        ("reverse", ctypes.c_int), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class GdnInProjParams(ctypes.Structure):
    """Mirror of ``gdn_in_proj_params`` in include/gdn.h."""
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("D", ctypes.c_int), ("C", ctypes.c_int),
        ("x", ctypes.c_void_p), ("w_in", ctypes.c_void_p), ("b_in", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("gate", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("log_a", ctypes.c_void_p),
    ]


class GdnOutProjParams(ctypes.Structure):
    """Mirror of ``gdn_out_proj_params`` in include/gdn.h."""
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("D", ctypes.c_int), ("C", ctypes.c_int),
        ("y", ctypes.c_void_p), ("w_out", ctypes.c_void_p), ("b_out", ctypes.c_void_p), ("out", ctypes.c_void_p),
    ]


class GdnMixerParams(ctypes.Structure):
    """Mirror of ``gdn_mixer_params`` in include/gdn.h."""
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("D", ctypes.c_int), ("C", ctypes.c_int),
        ("x", ctypes.c_void_p), ("w_in", ctypes.c_void_p), ("b_in", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
        ("conv_q", ctypes.c_void_p), ("conv_k", ctypes.c_void_p), ("conv_v", ctypes.c_void_p),
        ("norm_w", ctypes.c_void_p), ("eps_l2", ctypes.c_float), ("eps_norm", ctypes.c_float),
        ("S0", ctypes.c_void_p), ("S_T", ctypes.c_void_p), ("w_out", ctypes.c_void_p), ("b_out", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class GdnBwdParams(ctypes.Structure):
    """Mirror of ``gdn_bwd_params`` in include/gdn.h."""
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
        ("Dk", ctypes.c_int), ("Dv", ctypes.c_int), ("io_dtype", ctypes.c_int),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("log_a", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("gate", ctypes.c_void_p),
        ("conv_q", ctypes.c_void_p), ("conv_k", ctypes.c_void_p), ("conv_v", ctypes.c_void_p),
        ("norm_w", ctypes.c_void_p), ("eps_l2", ctypes.c_float), ("eps_norm", ctypes.c_float),
        ("S0", ctypes.c_void_p), ("dy", ctypes.c_void_p), ("dS_T", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p), ("dgate", ctypes.c_void_p),
        ("dlog_a", ctypes.c_void_p), ("dbeta", ctypes.c_void_p),
        ("dconv_q", ctypes.c_void_p), ("dconv_k", ctypes.c_void_p), ("dconv_v", ctypes.c_void_p),
        ("dnorm_w", ctypes.c_void_p), ("dS0", ctypes.c_void_p), ("reverse", ctypes.c_int),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gdn_status_string(status)} (status {status})")


_lib = None


def load(path: str | None = None):
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libgdn.so not built at {p}; run python -m linear_attention_token_fwd_amd.build")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(GdnFwdParams)
    lib.gdn_fwd.argtypes = [P, ctypes.c_void_p]
    lib.gdn_fwd.restype = ctypes.c_int
    lib.gdn_fwd_noalloc.argtypes = [P, ctypes.c_void_p]
    lib.gdn_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_fwd_bidir.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p]
    lib.gdn_fwd_bidir.restype = ctypes.c_int
    lib.gdn_fwd_workspace_bytes.argtypes = [P]
    lib.gdn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_fwd_bidir_workspace_bytes.argtypes = [P]
    lib.gdn_fwd_bidir_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_fwd_launch_count.argtypes = [P, ctypes.c_int]
    lib.gdn_fwd_launch_count.restype = ctypes.c_int
    lib.gdn_fwd_launch_name.argtypes = [P, ctypes.c_int, ctypes.c_int]
    lib.gdn_fwd_launch_name.restype = ctypes.c_char_p
    lib.gdn_fwd_timed.argtypes = [P, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                  ctypes.c_int, ctypes.c_void_p]
    lib.gdn_fwd_timed.restype = ctypes.c_int
    IP = ctypes.POINTER(ctypes.c_int)
    lib.gdn_fwd_varlen.argtypes = [P, IP, ctypes.c_void_p]
    lib.gdn_fwd_varlen.restype = ctypes.c_int
    lib.gdn_fwd_varlen_workspace_bytes.argtypes = [P, IP]
    lib.gdn_fwd_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_in_proj.argtypes = [ctypes.POINTER(GdnInProjParams), ctypes.c_void_p]
    lib.gdn_in_proj.restype = ctypes.c_int
    lib.gdn_out_proj.argtypes = [ctypes.POINTER(GdnOutProjParams), ctypes.c_void_p]
    lib.gdn_out_proj.restype = ctypes.c_int
    PM = ctypes.POINTER(GdnMixerParams)
    lib.gdn_mixer_workspace_bytes.argtypes = [PM]
    lib.gdn_mixer_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_mixer_fwd.argtypes = [PM, ctypes.c_void_p]
    lib.gdn_mixer_fwd.restype = ctypes.c_int
    lib.gdn_mixer_fwd_timed.argtypes = [PM, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_void_p]
    lib.gdn_mixer_fwd_timed.restype = ctypes.c_int
    PB = ctypes.POINTER(GdnBwdParams)
    lib.gdn_bwd_workspace_bytes.argtypes = [PB]
    lib.gdn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_bwd.argtypes = [PB, ctypes.c_void_p]
    lib.gdn_bwd.restype = ctypes.c_int
    lib.gdn_bwd_timed.argtypes = [PB, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_void_p]
    lib.gdn_bwd_timed.restype = ctypes.c_int
    lib.gdn_bwd_varlen.argtypes = [PB, IP, ctypes.c_void_p]
    lib.gdn_bwd_varlen.restype = ctypes.c_int
    lib.gdn_bwd_varlen_workspace_bytes.argtypes = [PB, IP]
    lib.gdn_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_bwd_launch_count.argtypes = []
    lib.gdn_bwd_launch_count.restype = ctypes.c_int
    lib.gdn_bwd_launch_name.argtypes = [ctypes.c_int]
    lib.gdn_bwd_launch_name.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_set_graph_cache_limit.argtypes = [ctypes.c_int]
    lib.gdn_set_graph_cache_limit.restype = ctypes.c_int
    lib.gdn_graph_cache_count.argtypes = []
    lib.gdn_graph_cache_count.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def gdn_status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


def gdn_set_graph_cache_limit(max_graphs: int) -> None:
    """Keep at most max_graphs recorded launch graphs (0 turns graphs off)."""
    st = load().gdn_set_graph_cache_limit(int(max_graphs))
    if st != GDN_OK:
        raise GdnError(st, "gdn_set_graph_cache_limit")


def gdn_graph_cache_count() -> int:
    """The number of launch graphs the library holds."""
    return int(load().gdn_graph_cache_count())


def _sizes(B, T, H, D, dtype) -> GdnFwdParams:
    p = GdnFwdParams()
    p.B, p.T, p.H, p.Dk, p.Dv = B, T, H, D, D
    p.io_dtype = dtype
    return p


def gdn_fwd_workspace_bytes(B: int, T: int, H: int, D: int, io_dtype: int = GDN_BF16) -> int:
    return load().gdn_fwd_workspace_bytes(ctypes.byref(_sizes(B, T, H, D, io_dtype)))


def gdn_fwd_bidir_workspace_bytes(B: int, T: int, H: int, D: int, io_dtype: int = GDN_BF16) -> int:
    return load().gdn_fwd_bidir_workspace_bytes(ctypes.byref(_sizes(B, T, H, D, io_dtype)))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, device):
    """The stream a call runs on: the given one, else the device's current stream."""
    import torch
    return stream if stream is not None else torch.cuda.current_stream(device)


def _alloc(shape, dtype, device, stream):
    """A tensor allocated on the pool of the stream the call runs on, so that
    the caching allocator reuses its memory only after that stream's work."""
    import torch
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes, device, stream):
    """The call's own workspace when the caller passes none: allocated on the
    call's stream (see _alloc), so freeing it on return is safe even when the
    call runs on a stream other than the current one."""
    import torch
    return _alloc((max(int(nbytes), 1),), torch.uint8, device, stream)


def _checked_table(cu_seqlens, total: int):
    """The sequence offsets as ints, after the checks the C layer cannot make
    (it does not see tensor sizes): offsets from 0, every length >= 1, and the
    last offset equal to the packed row count of the tensors."""
    vals = [int(x) for x in cu_seqlens]
    if len(vals) < 2:
        raise ValueError("cu_seqlens needs at least two offsets (one sequence)")
    if vals[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    if any(b <= a for a, b in zip(vals, vals[1:])):
        raise ValueError("cu_seqlens must increase: every sequence holds at least one token")
    if vals[-1] != int(total):
        raise ValueError(f"cu_seqlens ends at {vals[-1]}, but the tensors hold {total} token rows")
    return vals


def make_params(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T,
                workspace, eps_l2=1e-6, eps_norm=1e-6, reverse=False) -> GdnFwdParams:
    """Fill the params struct from torch tensors (no checks beyond shape
    reading: the library validates everything)."""
    import torch
    B, T, H, D = q.shape
    p = GdnFwdParams()
    p.B, p.T, p.H, p.Dk, p.Dv = B, T, H, D, v.shape[3]
    p.io_dtype = GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32
    p.q, p.k, p.v, p.gate = _ptr(q), _ptr(k), _ptr(v), _ptr(gate)
    p.log_a, p.beta = _ptr(log_a), _ptr(beta)
    p.conv_q, p.conv_k, p.conv_v = _ptr(conv_q), _ptr(conv_k), _ptr(conv_v)
    p.norm_w, p.S0 = _ptr(norm_w), _ptr(S0)
    p.eps_l2, p.eps_norm = eps_l2, eps_norm
    p.o, p.S_T = _ptr(out), _ptr(S_T)
    p.reverse = 1 if reverse else 0
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return p


def _check_all(specs):
    """_check over (tensor, name, dtype, shape) entries: dtype, shape and
    layout of every tensor first, then that each lives on the device."""
    for t, name, dt, shp in specs:
        _check(t, name, dt, shp, device=False)
    for t, name, dt, shp in specs:
        _check(t, name, dt, shp)


def _check(t, name, dtype, shape, device=True):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")


def _prepare(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T, stream=None):
    import torch
    B, T, H, D = q.shape
    io = q.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v, gate must be bfloat16 or float32")
    f32 = torch.float32
    _check_all(((q, "q", io, (B, T, H, D)), (k, "k", io, (B, T, H, D)),
                             (v, "v", io, (B, T, H, D)), (gate, "gate", io, (B, T, H, D)),
                             (log_a, "log_a", f32, (B, T, H)), (beta, "beta", f32, (B, T, H)),
                             (conv_q, "conv_q", f32, (H * D, 4)), (conv_k, "conv_k", f32, (H * D, 4)),
                             (conv_v, "conv_v", f32, (H * D, 4)), (norm_w, "norm_w", f32, (H, D)),
                             (S0, "S0", f32, (B, H, D, D)), (out, "out", io, (B, T, H, D)),
                             (S_T, "S_T", f32, (B, H, D, D))))
    if out is None:
        out = _alloc((B, T, H, D), io, q.device, _stream(stream, q.device))
    return out


def gdn_fwd(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w=None, S0=None,
            eps_l2=1e-6, eps_norm=1e-6, reverse=False, out=None, S_T=None, want_state=True,
            workspace=None, stream=None):
    """One GDN layer forward on device tensors.  Returns (out, S_T)."""
    import torch
    lib = load()
    strm = _stream(stream, q.device)
    out = _prepare(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T, strm)
    B, T, H, D = q.shape
    if S_T is None and want_state:
        S_T = _alloc((B, H, D, D), torch.float32, q.device, strm)
    need = gdn_fwd_workspace_bytes(B, T, H, D, GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32)
    if workspace is None:
        workspace = _workspace(need, q.device, strm)
    p = make_params(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T,
                    workspace, eps_l2, eps_norm, reverse)
    st = lib.gdn_fwd(ctypes.byref(p), ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_fwd")
    return out, S_T


def gdn_fwd_noalloc(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, out, S_T=None, norm_w=None, S0=None,
                    eps_l2=1e-6, eps_norm=1e-6, reverse=False, stream=None):
    """gdn_fwd into caller-given outputs (out, and S_T or None) with the
    library's own 64 MiB device workspace: nothing is allocated, by the
    binding or by the library.  Returns (out, S_T)."""
    lib = load()
    strm = _stream(stream, q.device)
    _prepare(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T, strm)
    if out is None:
        raise ValueError("gdn_fwd_noalloc writes into a caller-given out tensor")
    p = make_params(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T, None,
                    eps_l2, eps_norm, reverse)
    st = lib.gdn_fwd_noalloc(ctypes.byref(p), ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_fwd_noalloc")
    return out, S_T


def gdn_fwd_bidir(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w=None, S0=None,
                  eps_l2=1e-6, eps_norm=1e-6, out=None, S_T=None, S_T_rev=None, want_state=True,
                  workspace=None, stream=None):
    """Forward and time-reversed scans, outputs added.  Returns (out, S_T, S_T_rev)."""
    import torch
    lib = load()
    strm = _stream(stream, q.device)
    out = _prepare(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T, strm)
    B, T, H, D = q.shape
    _check(S_T_rev, "S_T_rev", torch.float32, (B, H, D, D))
    if want_state:
        if S_T is None:
            S_T = _alloc((B, H, D, D), torch.float32, q.device, strm)
        if S_T_rev is None:
            S_T_rev = _alloc((B, H, D, D), torch.float32, q.device, strm)
    need = gdn_fwd_bidir_workspace_bytes(B, T, H, D, GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32)
    if workspace is None:
        workspace = _workspace(need, q.device, strm)
    p = make_params(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T,
                    workspace, eps_l2, eps_norm, False)
    st = lib.gdn_fwd_bidir(ctypes.byref(p), ctypes.c_void_p(_ptr(S_T_rev)), ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_fwd_bidir")
    return out, S_T, S_T_rev


def to_device(inp: dict, device="cuda", dtype=None):
    """Move a seeded input dict (float32 numpy arrays holding exact values) to
    device tensors: q, k, v, gate in the workload's I/O dtype, the rest fp32."""
    import torch
    out = {}
    for key, val in inp.items():
        if val is None:
            out[key] = None
            continue
        t = torch.from_numpy(val)
        if key in ("q", "k", "v", "gate") and dtype is not None:
            t = t.to(dtype)
        out[key] = t.to(device).contiguous()
    return out


def in_proj_params(x, w_in, b_in, A_log, H, D, q, k, v, gate, beta, log_a) -> GdnInProjParams:
    """Fill the in-projection params struct from torch tensors (the library
    validates everything)."""
    B, T, C = x.shape
    p = GdnInProjParams()
    p.B, p.T, p.H, p.D, p.C = B, T, H, D, C
    p.x, p.w_in, p.b_in, p.A_log = _ptr(x), _ptr(w_in), _ptr(b_in), _ptr(A_log)
    p.q, p.k, p.v, p.gate = _ptr(q), _ptr(k), _ptr(v), _ptr(gate)
    p.beta, p.log_a = _ptr(beta), _ptr(log_a)
    return p


def gdn_in_proj(x, w_in, A_log, H, D, b_in=None, stream=None):
    """q, k, v, gate ([B, T, H, D] bf16) and beta, log_a ([B, T, H] fp32) from
    the hidden states x [B, T, C] bf16 and the stacked weight
    w_in [4 H D + 2 H, C] bf16.  Returns (q, k, v, gate, beta, log_a)."""
    import torch
    B, T, C = x.shape
    N = 4 * H * D + 2 * H
    _check(x, "x", torch.bfloat16, (B, T, C))
    _check(w_in, "w_in", torch.bfloat16, (N, C))
    _check(b_in, "b_in", torch.float32, (N,))
    _check(A_log, "A_log", torch.float32, (H,))
    dev = x.device
    strm = _stream(stream, dev)
    q, k, v, gate = (_alloc((B, T, H, D), torch.bfloat16, dev, strm) for _ in range(4))
    beta = _alloc((B, T, H), torch.float32, dev, strm)
    log_a = _alloc((B, T, H), torch.float32, dev, strm)
    p = in_proj_params(x, w_in, b_in, A_log, H, D, q, k, v, gate, beta, log_a)
    st = load().gdn_in_proj(ctypes.byref(p), ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_in_proj")
    return q, k, v, gate, beta, log_a


def out_proj_params(y, w_out, b_out, out) -> GdnOutProjParams:
    B, T, H, D = y.shape
    p = GdnOutProjParams()
    p.B, p.T, p.H, p.D, p.C = B, T, H, D, w_out.shape[0]
    p.y, p.w_out, p.b_out, p.out = _ptr(y), _ptr(w_out), _ptr(b_out), _ptr(out)
    return p


def gdn_out_proj(y, w_out, b_out=None, out=None, stream=None):
    """out [B, T, C] bf16 = y [B, T, H, D] (as [B T, H D]) times w_out^T
    ([C, H D] bf16) plus b_out."""
    import torch
    B, T, H, D = y.shape
    C = w_out.shape[0]
    _check(y, "y", torch.bfloat16, (B, T, H, D))
    _check(w_out, "w_out", torch.bfloat16, (C, H * D))
    _check(b_out, "b_out", torch.float32, (C,))
    _check(out, "out", torch.bfloat16, (B, T, C))
    strm = _stream(stream, y.device)
    if out is None:
        out = _alloc((B, T, C), torch.bfloat16, y.device, strm)
    p = out_proj_params(y, w_out, b_out, out)
    st = load().gdn_out_proj(ctypes.byref(p), ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_out_proj")
    return out


def mixer_params(x, w_in, b_in, A_log, conv_q, conv_k, conv_v, norm_w, S0, w_out, b_out, out, S_T,
                 workspace, H, D, eps_l2=1e-6, eps_norm=1e-6) -> GdnMixerParams:
    """Fill the mixer params struct from torch tensors (the library validates)."""
    B, T, C = x.shape
    p = GdnMixerParams()
    p.B, p.T, p.H, p.D, p.C = B, T, H, D, C
    p.x, p.w_in, p.b_in, p.A_log = _ptr(x), _ptr(w_in), _ptr(b_in), _ptr(A_log)
    p.conv_q, p.conv_k, p.conv_v, p.norm_w = _ptr(conv_q), _ptr(conv_k), _ptr(conv_v), _ptr(norm_w)
    p.eps_l2, p.eps_norm = eps_l2, eps_norm
    p.S0, p.S_T, p.w_out, p.b_out, p.out = _ptr(S0), _ptr(S_T), _ptr(w_out), _ptr(b_out), _ptr(out)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return p


def gdn_mixer_workspace_bytes(B: int, T: int, H: int, D: int, C: int) -> int:
    p = GdnMixerParams()
    p.B, p.T, p.H, p.D, p.C = B, T, H, D, C
    return load().gdn_mixer_workspace_bytes(ctypes.byref(p))


def gdn_mixer_fwd(x, w_in, A_log, conv_q, conv_k, conv_v, w_out, H, D, b_in=None, b_out=None, norm_w=None,
                  S0=None, eps_l2=1e-6, eps_norm=1e-6, out=None, S_T=None, want_state=True, workspace=None,
                  stream=None):
    """The whole token mixer on device tensors: out [B, T, C] bf16 =
    out_proj(GDN layer(in_proj(x))).  Returns (out, S_T)."""
    import torch
    B, T, C = x.shape
    N = 4 * H * D + 2 * H
    f32 = torch.float32
    _check_all(((x, "x", torch.bfloat16, (B, T, C)), (w_in, "w_in", torch.bfloat16, (N, C)),
                             (b_in, "b_in", f32, (N,)), (A_log, "A_log", f32, (H,)),
                             (conv_q, "conv_q", f32, (H * D, 4)), (conv_k, "conv_k", f32, (H * D, 4)),
                             (conv_v, "conv_v", f32, (H * D, 4)), (norm_w, "norm_w", f32, (H, D)),
                             (S0, "S0", f32, (B, H, D, D)), (w_out, "w_out", torch.bfloat16, (C, H * D)),
                             (b_out, "b_out", f32, (C,)), (out, "out", torch.bfloat16, (B, T, C)),
                             (S_T, "S_T", f32, (B, H, D, D))))
    strm = _stream(stream, x.device)
    if out is None:
        out = _alloc((B, T, C), torch.bfloat16, x.device, strm)
    if S_T is None and want_state:
        S_T = _alloc((B, H, D, D), f32, x.device, strm)
    if workspace is None:
        workspace = _workspace(gdn_mixer_workspace_bytes(B, T, H, D, C), x.device, strm)
    p = mixer_params(x, w_in, b_in, A_log, conv_q, conv_k, conv_v, norm_w, S0, w_out, b_out, out, S_T,
                     workspace, H, D, eps_l2, eps_norm)
    st = load().gdn_mixer_fwd(ctypes.byref(p), ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_mixer_fwd")
    return out, S_T


def seq_table(cu_seqlens):
    """A ctypes int array of the sequence offsets (host memory)."""
    vals = [int(x) for x in cu_seqlens]
    return (ctypes.c_int * len(vals))(*vals)


def gdn_fwd_varlen_workspace_bytes(cu_seqlens, H: int, D: int, io_dtype: int = GDN_BF16) -> int:
    cu = seq_table(cu_seqlens)
    return load().gdn_fwd_varlen_workspace_bytes(ctypes.byref(_sizes(len(cu) - 1, 0, H, D, io_dtype)), cu)


def gdn_fwd_varlen(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, cu_seqlens, norm_w=None, S0=None,
                   eps_l2=1e-6, eps_norm=1e-6, reverse=False, out=None, S_T=None, want_state=True,
                   workspace=None, stream=None):
    """A variable-length batch: q, k, v, gate [1, total, H, D], log_a, beta
    [1, total, H], sequences at token rows cu_seqlens[b] .. cu_seqlens[b+1]-1
    (a host sequence of ints), S0 / S_T [N, H, D, D].  Returns (out, S_T)."""
    import torch
    lib = load()
    if not isinstance(q, torch.Tensor) or q.dim() != 4 or q.shape[0] != 1:
        raise ValueError("q must be [1, total, H, D] (sequences packed along the token axis)")
    cu = seq_table(_checked_table(cu_seqlens, q.shape[1]))
    N = len(cu) - 1
    strm = _stream(stream, q.device)
    out = _prepare(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, None, out, None, strm)
    _, total, H, D = q.shape
    _check(S0, "S0", torch.float32, (N, H, D, D))
    _check(S_T, "S_T", torch.float32, (N, H, D, D))
    if S_T is None and want_state:
        S_T = _alloc((N, H, D, D), torch.float32, q.device, strm)
    io = GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32
    if workspace is None:
        need = lib.gdn_fwd_varlen_workspace_bytes(ctypes.byref(_sizes(N, 0, H, D, io)), cu)
        workspace = _workspace(need, q.device, strm)
    p = make_params(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, out, S_T, workspace,
                    eps_l2, eps_norm, reverse)
    p.B = N
    st = lib.gdn_fwd_varlen(ctypes.byref(p), cu, ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_fwd_varlen")
    return out, S_T


# ---- backward pass

BWD_GRADS = ("q", "k", "v", "log_a", "beta", "gate", "conv_q", "conv_k", "conv_v", "norm_w", "S0")


def gdn_bwd_workspace_bytes(B: int, T: int, H: int, D: int, io_dtype: int = GDN_BF16) -> int:
    p = GdnBwdParams()
    p.B, p.T, p.H, p.Dk, p.Dv, p.io_dtype = B, T, H, D, D, io_dtype
    return load().gdn_bwd_workspace_bytes(ctypes.byref(p))


def gdn_bwd_launch_names() -> list:
    lib = load()
    return [lib.gdn_bwd_launch_name(i).decode() for i in range(lib.gdn_bwd_launch_count())]


def bwd_params(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, dy, dS_T, grads: dict,
               workspace, eps_l2=1e-6, eps_norm=1e-6, reverse=False) -> GdnBwdParams:
    """Fill the backward params struct from torch tensors; grads maps the
    names of BWD_GRADS to output tensors (norm_w and S0 may be None)."""
    import torch
    B, T, H, D = q.shape
    p = GdnBwdParams()
    p.B, p.T, p.H, p.Dk, p.Dv = B, T, H, D, v.shape[3]
    p.io_dtype = GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32
    p.q, p.k, p.v, p.gate = _ptr(q), _ptr(k), _ptr(v), _ptr(gate)
    p.log_a, p.beta = _ptr(log_a), _ptr(beta)
    p.conv_q, p.conv_k, p.conv_v = _ptr(conv_q), _ptr(conv_k), _ptr(conv_v)
    p.norm_w, p.S0 = _ptr(norm_w), _ptr(S0)
    p.eps_l2, p.eps_norm = eps_l2, eps_norm
    p.dy, p.dS_T = _ptr(dy), _ptr(dS_T)
    p.dq, p.dk, p.dv, p.dgate = (_ptr(grads.get(n)) for n in ("q", "k", "v", "gate"))
    p.dlog_a, p.dbeta = _ptr(grads.get("log_a")), _ptr(grads.get("beta"))
    p.dconv_q, p.dconv_k, p.dconv_v = (_ptr(grads.get(n)) for n in ("conv_q", "conv_k", "conv_v"))
    p.dnorm_w, p.dS0 = _ptr(grads.get("norm_w")), _ptr(grads.get("S0"))
    p.reverse = 1 if reverse else 0
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return p


def gdn_bwd(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, dy, dS_T=None,
            eps_l2=1e-6, eps_norm=1e-6, want_norm_w=True, want_S0=True, out=None, workspace=None,
            stream=None, reverse=False):
    """Gradients of the layer forward (with the same reverse flag) given dy
    (and dS_T, the final state's gradient, or None).  Returns a dict keyed by BWD_GRADS:
    dq, dk, dv, dgate in the I/O dtype, the rest float32 (norm_w / S0: None
    unless wanted).  out: an optional dict of preallocated output tensors
    under the same keys."""
    import torch
    lib = load()
    _prepare(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, None, None)
    B, T, H, D = q.shape
    _check(dy, "dy", q.dtype, (B, T, H, D))
    _check(dS_T, "dS_T", torch.float32, (B, H, D, D))
    dev, io, f32 = q.device, q.dtype, torch.float32
    strm = _stream(stream, dev)
    g = {n: _alloc((B, T, H, D), io, dev, strm) for n in ("q", "k", "v", "gate")}
    g["log_a"] = _alloc((B, T, H), f32, dev, strm)
    g["beta"] = _alloc((B, T, H), f32, dev, strm)
    for n in ("conv_q", "conv_k", "conv_v"):
        g[n] = _alloc((H * D, 4), f32, dev, strm)
    g["norm_w"] = _alloc((H, D), f32, dev, strm) if want_norm_w else None
    g["S0"] = _alloc((B, H, D, D), f32, dev, strm) if want_S0 else None
    if out is not None:
        for n, t in out.items():
            if g.get(n) is not None:
                _check(t, "d" + n, g[n].dtype, tuple(g[n].shape))
            g[n] = t
    need = gdn_bwd_workspace_bytes(B, T, H, D, GDN_BF16 if io == torch.bfloat16 else GDN_F32)
    if workspace is None:
        workspace = _workspace(need, dev, strm)
    p = bwd_params(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, dy, dS_T, g,
                   workspace, eps_l2, eps_norm, reverse)
    st = lib.gdn_bwd(ctypes.byref(p), ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_bwd")
    return g


def gdn_bwd_varlen(q, k, v, log_a, beta, gate, conv_q, conv_k, conv_v, norm_w, S0, dy, dS_T, cu_seqlens,
                   eps_l2=1e-6, eps_norm=1e-6, want_norm_w=True, want_S0=True, reverse=False, stream=None):
    """The backward of gdn_fwd_varlen: q, k, v, gate, dy [total, H, D] (a
    leading batch dimension of 1 is accepted), log_a, beta [total, H] (or
    [1, total, H]); cu_seqlens a host sequence of B + 1 ints; S0, dS_T
    [B, H, D, D] or None.  Returns a dict keyed by BWD_GRADS (per-token
    gradients shaped like their inputs).  Every tensor is checked (device,
    dtype, shape, contiguity) and the table against the packed row count
    before anything is launched."""
    import torch
    lib = load()
    if not isinstance(q, torch.Tensor) or q.dim() not in (3, 4) or (q.dim() == 4 and q.shape[0] != 1):
        raise ValueError("q must be [total, H, D] or [1, total, H, D]")
    total, H, D = tuple(q.shape[-3:])
    vals = _checked_table(cu_seqlens, total)
    cu = seq_table(vals)
    B = len(vals) - 1
    dev, io, f32 = q.device, q.dtype, torch.float32
    if io not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v, gate, dy must be bfloat16 or float32")
    tok_shape = tuple(q.shape)
    gate_shape = tuple(log_a.shape) if isinstance(log_a, torch.Tensor) else None
    if gate_shape not in ((total, H), (1, total, H)):
        raise ValueError(f"log_a must be [total, H] or [1, total, H], got {gate_shape}")
    _check_all(((q, "q", io, tok_shape), (k, "k", io, tok_shape), (v, "v", io, tok_shape),
                             (gate, "gate", io, tok_shape), (dy, "dy", io, tok_shape),
                             (log_a, "log_a", f32, gate_shape), (beta, "beta", f32, gate_shape),
                             (conv_q, "conv_q", f32, (H * D, 4)), (conv_k, "conv_k", f32, (H * D, 4)),
                             (conv_v, "conv_v", f32, (H * D, 4)), (norm_w, "norm_w", f32, (H, D)),
                             (S0, "S0", f32, (B, H, D, D)), (dS_T, "dS_T", f32, (B, H, D, D))))
    strm = _stream(stream, dev)
    g = {n: _alloc(tok_shape, io, dev, strm) for n in ("q", "k", "v", "gate")}
    g["log_a"] = _alloc(gate_shape, f32, dev, strm)
    g["beta"] = _alloc(gate_shape, f32, dev, strm)
    for n in ("conv_q", "conv_k", "conv_v"):
        g[n] = _alloc((H * D, 4), f32, dev, strm)
    g["norm_w"] = _alloc((H, D), f32, dev, strm) if want_norm_w else None
    g["S0"] = _alloc((B, H, D, D), f32, dev, strm) if want_S0 else None
    p = GdnBwdParams()
    p.B, p.T, p.H, p.Dk, p.Dv = B, 0, H, D, D
    p.io_dtype = GDN_BF16 if io == torch.bfloat16 else GDN_F32
    need = lib.gdn_bwd_varlen_workspace_bytes(ctypes.byref(p), cu)
    if need == 0:
        raise GdnError(GDN_ERR_INVALID_ARG, "gdn_bwd_varlen_workspace_bytes")
    workspace = _workspace(need, dev, strm)
    def as4(t):
        return t.reshape(1, total, H, D)
    p = bwd_params(as4(q), as4(k), as4(v), log_a, beta, as4(gate), conv_q, conv_k, conv_v, norm_w, S0, as4(dy),
                   dS_T, g, workspace, eps_l2, eps_norm, reverse)
    p.B, p.T = B, 0
    st = lib.gdn_bwd_varlen(ctypes.byref(p), cu, ctypes.c_void_p(strm.cuda_stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_bwd_varlen")
    return g

"""The C ABI of libgdn.so on the host (no GPU needed).

* Every function include/gdn.h declares is exported by the library and bound
  by the Python binding.
* The host-side logic answers without touching a GPU: status strings, sizes,
  workspace sizes, the launch plan, and every validation error.  Validation
  only looks at pointer values and sizes, so the error cases below use fake,
  never dereferenced device addresses; each case fails validation before the
  first HIP call.
"""
import ctypes
import math
import os
import re

import pytest

import linear_attention_token_fwd_amd as gdn

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "gdn.h")


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:gdn_status|size_t|int|const\s+char\s*\*)\s*(gdn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built: run python -m linear_attention_token_fwd_amd.build")
    return gdn.load()


def test_every_declared_function_is_exported_and_bound(lib):
    decl = declared_functions()
    assert len(decl) == 25, decl
    assert set(decl) == set(gdn.EXPORTS)
    for name in decl:
        fn = getattr(lib, name)  # AttributeError if the library does not export it
        assert fn.argtypes is not None, name  # bound by the binding


def test_missing_library_fails_loudly():
    with pytest.raises(RuntimeError):
        gdn.load("/nonexistent/libgdn.so")


def test_status_strings(lib):
    texts = [lib.gdn_status_string(s).decode() for s in range(6)]
    assert all(texts) and len(set(texts)) == 6
    assert lib.gdn_status_string(99)  # unknown codes still get text


def test_graph_cache_limit(lib):
    assert lib.gdn_set_graph_cache_limit(-1) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_set_graph_cache_limit(65) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_set_graph_cache_limit(0) == gdn.GDN_OK
    assert lib.gdn_set_graph_cache_limit(8) == gdn.GDN_OK
    assert lib.gdn_graph_cache_count() == 0  # nothing is recorded without a device call
    with pytest.raises(gdn.GdnError):
        gdn.gdn_set_graph_cache_limit(100)


BF16_W1 = (1, 32760, 12, 128, gdn.GDN_BF16)


def test_workspace_sizes(lib):
    B, T, H, D, io = BF16_W1
    ws = gdn.gdn_fwd_workspace_bytes(B, T, H, D, io)
    NC = math.ceil(T / 64)
    records = B * H * NC * 320 * D * 2   # -W, Q', (D K)^T, U~, O0 per chunk-head
    states = B * H * NC * D * D * 2      # chunk-entry states
    assert records + states <= ws <= records + states + 64 * 2**20
    assert gdn.gdn_fwd_bidir_workspace_bytes(B, T, H, D, io) >= 2 * ws
    assert gdn.gdn_fwd_workspace_bytes(B, 2 * T, H, D, io) > ws
    for bad in ((0, T, H, D, io), (B, 0, H, D, io), (B, T, 0, D, io), (B, T, H, D, 7)):
        assert gdn.gdn_fwd_workspace_bytes(*bad) == 0


def test_launch_plan(lib):
    B, T, H, D, io = BF16_W1
    p = gdn._sizes(B, T, H, D, io)
    n = lib.gdn_fwd_launch_count(ctypes.byref(p), 0)
    names = [lib.gdn_fwd_launch_name(ctypes.byref(p), 0, i).decode() for i in range(n)]
    ranges = n // 3
    assert n == 3 * ranges and ranges >= 2
    assert names == ["gdn_prep_kernel"] * ranges + ["gdn_state_kernel"] * ranges + ["gdn_out_kernel"] * ranges
    assert lib.gdn_fwd_launch_name(ctypes.byref(p), 0, n) is None
    # both scans: prep, state and output per range and direction, with longer
    # ranges (about 400 chunks against about 170 for one scan)
    NC = math.ceil(T / 64)
    assert ranges == math.ceil(NC / 170)
    assert lib.gdn_fwd_launch_count(ctypes.byref(p), 1) == 2 * 3 * math.ceil(NC / 400)
    short = gdn._sizes(1, 100, 2, 64, gdn.GDN_F32)
    assert lib.gdn_fwd_launch_count(ctypes.byref(short), 0) == 3
    for unsupported in ((1, 64, 2, 96, gdn.GDN_BF16), (1, 64, 2, 32, gdn.GDN_F32)):
        assert lib.gdn_fwd_launch_count(ctypes.byref(gdn._sizes(*unsupported)), 0) == -1
    # every I/O dtype with D = 64 and D = 128
    for io in (gdn.GDN_BF16, gdn.GDN_F32):
        for D in (64, 128):
            assert lib.gdn_fwd_launch_count(ctypes.byref(gdn._sizes(1, 100, 2, D, io)), 0) == 3


def fake_params(lib, B=1, T=200, H=2, D=64, io=gdn.GDN_BF16, bidir=False):
    """A params struct whose buffers are distinct, aligned, non-overlapping
    fake device addresses, with a large enough workspace."""
    p = gdn._sizes(B, T, H, D, io)
    base, step = 1 << 44, 1 << 36
    names = ["q", "k", "v", "log_a", "beta", "gate", "conv_q", "conv_k", "conv_v", "norm_w", "S0", "o", "S_T",
             "workspace"]
    for i, nm in enumerate(names):
        setattr(p, nm, base + i * step)
    p.eps_l2 = p.eps_norm = 1e-6
    p.reverse = 0
    p.workspace_bytes = (lib.gdn_fwd_bidir_workspace_bytes if bidir else lib.gdn_fwd_workspace_bytes)(ctypes.byref(p))
    assert p.workspace_bytes > 0
    return p


def status_of(lib, p):
    return lib.gdn_fwd(ctypes.byref(p), None)


CASES = [
    ("q NULL", lambda p: setattr(p, "q", None), gdn.GDN_ERR_INVALID_ARG),
    ("gate NULL", lambda p: setattr(p, "gate", None), gdn.GDN_ERR_INVALID_ARG),
    ("output NULL", lambda p: setattr(p, "o", None), gdn.GDN_ERR_INVALID_ARG),
    ("eps_l2 < 0", lambda p: setattr(p, "eps_l2", -1.0), gdn.GDN_ERR_INVALID_ARG),
    ("eps_norm NaN", lambda p: setattr(p, "eps_norm", float("nan")), gdn.GDN_ERR_INVALID_ARG),
    ("reverse = 2", lambda p: setattr(p, "reverse", 2), gdn.GDN_ERR_INVALID_ARG),
    ("T = 0", lambda p: setattr(p, "T", 0), gdn.GDN_ERR_INVALID_ARG),
    ("Dk != Dv", lambda p: setattr(p, "Dv", 128), gdn.GDN_ERR_UNSUPPORTED),
    ("D = 96", lambda p: (setattr(p, "Dk", 96), setattr(p, "Dv", 96)), gdn.GDN_ERR_UNSUPPORTED),
    ("fp32 D = 64, Dv = 128", lambda p: (setattr(p, "io_dtype", gdn.GDN_F32), setattr(p, "Dv", 128)),
     gdn.GDN_ERR_UNSUPPORTED),
    ("q misaligned", lambda p: setattr(p, "q", p.q + 8), gdn.GDN_ERR_ALIGNMENT),
    ("log_a misaligned", lambda p: setattr(p, "log_a", p.log_a + 2), gdn.GDN_ERR_ALIGNMENT),
    ("workspace NULL", lambda p: setattr(p, "workspace", None), gdn.GDN_ERR_WORKSPACE),
    ("workspace too small", lambda p: setattr(p, "workspace_bytes", p.workspace_bytes - 1), gdn.GDN_ERR_WORKSPACE),
    ("workspace misaligned", lambda p: setattr(p, "workspace", p.workspace + 16), gdn.GDN_ERR_ALIGNMENT),
    ("output overlaps q", lambda p: setattr(p, "o", p.q + 256), gdn.GDN_ERR_INVALID_ARG),
    ("S_T overlaps the workspace", lambda p: setattr(p, "S_T", p.workspace + 4096), gdn.GDN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,mutate,expect", CASES, ids=[c[0] for c in CASES])
def test_validation_errors(lib, name, mutate, expect):
    p = fake_params(lib)
    mutate(p)
    assert status_of(lib, p) == expect, name


def test_bidirectional_rejects_reverse(lib):
    p = fake_params(lib, bidir=True)
    p.reverse = 1
    assert lib.gdn_fwd_bidir(ctypes.byref(p), None, None) == gdn.GDN_ERR_INVALID_ARG


def test_timed_call_needs_two_events_per_launch(lib):
    p = fake_params(lib)
    n = lib.gdn_fwd_launch_count(ctypes.byref(p), 0)
    events = (ctypes.c_void_p * (2 * n - 1))()
    st = lib.gdn_fwd_timed(ctypes.byref(p), None, 0, events, 2 * n - 1, None)
    assert st == gdn.GDN_ERR_INVALID_ARG


def fake_in_proj(B=1, T=300, H=3, D=64, C=192):
    """In-projection params on distinct, aligned, fake device addresses."""
    p = gdn.GdnInProjParams()
    p.B, p.T, p.H, p.D, p.C = B, T, H, D, C
    base, step = 1 << 44, 1 << 36
    for i, nm in enumerate(["x", "w_in", "b_in", "A_log", "q", "k", "v", "gate", "beta", "log_a"]):
        setattr(p, nm, base + i * step)
    return p


def fake_out_proj(B=1, T=300, H=3, D=64, C=192):
    p = gdn.GdnOutProjParams()
    p.B, p.T, p.H, p.D, p.C = B, T, H, D, C
    base, step = 1 << 44, 1 << 36
    for i, nm in enumerate(["y", "w_out", "b_out", "out"]):
        setattr(p, nm, base + i * step)
    return p


IN_PROJ_CASES = [
    ("x NULL", lambda p: setattr(p, "x", None), gdn.GDN_ERR_INVALID_ARG),
    ("A_log NULL", lambda p: setattr(p, "A_log", None), gdn.GDN_ERR_INVALID_ARG),
    ("log_a NULL", lambda p: setattr(p, "log_a", None), gdn.GDN_ERR_INVALID_ARG),
    ("T = 0", lambda p: setattr(p, "T", 0), gdn.GDN_ERR_INVALID_ARG),
    ("C % 64 != 0", lambda p: setattr(p, "C", 160), gdn.GDN_ERR_UNSUPPORTED),
    ("H D % 16 != 0", lambda p: setattr(p, "D", 60), gdn.GDN_ERR_UNSUPPORTED),
    ("x too large", lambda p: (setattr(p, "T", 1 << 22), setattr(p, "C", 1024)), gdn.GDN_ERR_UNSUPPORTED),
    ("w_in misaligned", lambda p: setattr(p, "w_in", p.w_in + 8), gdn.GDN_ERR_ALIGNMENT),
    ("b_in misaligned", lambda p: setattr(p, "b_in", p.b_in + 4), gdn.GDN_ERR_ALIGNMENT),
    ("beta misaligned", lambda p: setattr(p, "beta", p.beta + 2), gdn.GDN_ERR_ALIGNMENT),
    ("q over x", lambda p: setattr(p, "q", p.x + 256), gdn.GDN_ERR_INVALID_ARG),
    ("gate over k", lambda p: setattr(p, "gate", p.k + 1024), gdn.GDN_ERR_INVALID_ARG),
    ("log_a over the bias", lambda p: setattr(p, "log_a", p.b_in), gdn.GDN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,mutate,expect", IN_PROJ_CASES, ids=[c[0] for c in IN_PROJ_CASES])
def test_in_proj_validation(lib, name, mutate, expect):
    p = fake_in_proj()
    mutate(p)
    assert lib.gdn_in_proj(ctypes.byref(p), None) == expect, name


OUT_PROJ_CASES = [
    ("y NULL", lambda p: setattr(p, "y", None), gdn.GDN_ERR_INVALID_ARG),
    ("out NULL", lambda p: setattr(p, "out", None), gdn.GDN_ERR_INVALID_ARG),
    ("C = 0", lambda p: setattr(p, "C", 0), gdn.GDN_ERR_INVALID_ARG),
    ("H D % 64 != 0", lambda p: setattr(p, "D", 48), gdn.GDN_ERR_UNSUPPORTED),
    ("C % 8 != 0", lambda p: setattr(p, "C", 196), gdn.GDN_ERR_UNSUPPORTED),
    ("w_out misaligned", lambda p: setattr(p, "w_out", p.w_out + 2), gdn.GDN_ERR_ALIGNMENT),
    ("out over y", lambda p: setattr(p, "out", p.y + 16), gdn.GDN_ERR_INVALID_ARG),
    ("out over w_out", lambda p: setattr(p, "out", p.w_out), gdn.GDN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,mutate,expect", OUT_PROJ_CASES, ids=[c[0] for c in OUT_PROJ_CASES])
def test_out_proj_validation(lib, name, mutate, expect):
    p = fake_out_proj()
    mutate(p)
    assert lib.gdn_out_proj(ctypes.byref(p), None) == expect, name


def test_projection_params_null():
    lib = gdn.load()
    assert lib.gdn_in_proj(None, None) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_out_proj(None, None) == gdn.GDN_ERR_INVALID_ARG


def fake_mixer(lib, B=1, T=300, H=3, D=64, C=192):
    p = gdn.GdnMixerParams()
    p.B, p.T, p.H, p.D, p.C = B, T, H, D, C
    base, step = 1 << 44, 1 << 36
    names = ["x", "w_in", "b_in", "A_log", "conv_q", "conv_k", "conv_v", "norm_w", "S0", "S_T", "w_out", "b_out",
             "out", "workspace"]
    for i, nm in enumerate(names):
        setattr(p, nm, base + i * step)
    p.eps_l2 = p.eps_norm = 1e-6
    p.workspace_bytes = lib.gdn_mixer_workspace_bytes(ctypes.byref(p))
    return p


def test_mixer_workspace_bytes(lib):
    B, T, H, D, C = 1, 32760, 12, 128, 1536
    need = gdn.gdn_mixer_workspace_bytes(B, T, H, D, C)
    inter = 5 * B * T * H * D * 2 + 2 * B * T * H * 4  # q, k, v, gate, y and b, log a
    layer = gdn.gdn_fwd_workspace_bytes(B, T, H, D, gdn.GDN_BF16)
    assert inter + layer <= need <= inter + layer + 8 * 256
    assert gdn.gdn_mixer_workspace_bytes(0, T, H, D, C) == 0


MIXER_CASES = [
    ("x NULL", lambda p: setattr(p, "x", None), gdn.GDN_ERR_INVALID_ARG),
    ("conv_k NULL", lambda p: setattr(p, "conv_k", None), gdn.GDN_ERR_INVALID_ARG),
    ("w_out NULL", lambda p: setattr(p, "w_out", None), gdn.GDN_ERR_INVALID_ARG),
    ("D = 96", lambda p: setattr(p, "D", 96), gdn.GDN_ERR_WORKSPACE),
    ("C % 64 != 0", lambda p: setattr(p, "C", 160), gdn.GDN_ERR_UNSUPPORTED),
    ("eps negative", lambda p: setattr(p, "eps_norm", -1.0), gdn.GDN_ERR_INVALID_ARG),
    ("workspace NULL", lambda p: setattr(p, "workspace", None), gdn.GDN_ERR_WORKSPACE),
    ("workspace small", lambda p: setattr(p, "workspace_bytes", p.workspace_bytes - 1), gdn.GDN_ERR_WORKSPACE),
    ("workspace misaligned", lambda p: setattr(p, "workspace", p.workspace + 64), gdn.GDN_ERR_ALIGNMENT),
    ("S0 inside the workspace", lambda p: setattr(p, "S0", p.workspace + 1024), gdn.GDN_ERR_INVALID_ARG),
    ("out over x", lambda p: setattr(p, "out", p.x + 512), gdn.GDN_ERR_INVALID_ARG),
    ("S_T over w_out", lambda p: setattr(p, "S_T", p.w_out), gdn.GDN_ERR_INVALID_ARG),
    ("S_T over out", lambda p: setattr(p, "S_T", p.out + 4096), gdn.GDN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,mutate,expect", MIXER_CASES, ids=[c[0] for c in MIXER_CASES])
def test_mixer_validation(lib, name, mutate, expect):
    p = fake_mixer(lib)
    mutate(p)
    assert lib.gdn_mixer_fwd(ctypes.byref(p), None) == expect, name


def test_mixer_timed_needs_events(lib):
    p = fake_mixer(lib)
    assert lib.gdn_mixer_fwd_timed(ctypes.byref(p), None, 0, None) == gdn.GDN_ERR_INVALID_ARG
    n = lib.gdn_fwd_launch_count(ctypes.byref(gdn._sizes(1, 300, 3, 64, gdn.GDN_BF16)), 0)
    events = (ctypes.c_void_p * (3 + 2 * n))()
    assert lib.gdn_mixer_fwd_timed(ctypes.byref(p), events, 3 + 2 * n, None) == gdn.GDN_ERR_INVALID_ARG


def test_varlen_workspace_and_table_checks(lib):
    p = fake_params(lib, B=3, T=1, H=2, D=64)
    good = gdn.seq_table([0, 5, 70, 200])
    need = lib.gdn_fwd_varlen_workspace_bytes(ctypes.byref(p), good)
    # as a batch of 3 rows of the longest length (130), plus the table
    dense = gdn.gdn_fwd_workspace_bytes(3, 130, 2, 64, gdn.GDN_BF16)
    assert dense < need <= dense + 256
    for bad in ([1, 5, 70, 200], [0, 5, 5, 200], [0, 70, 5, 200]):
        assert lib.gdn_fwd_varlen_workspace_bytes(ctypes.byref(p), gdn.seq_table(bad)) == 0
    assert lib.gdn_fwd_varlen_workspace_bytes(ctypes.byref(p), None) == 0


def test_varlen_validation(lib):
    p = fake_params(lib, B=3, T=1, H=2, D=64)
    cu = gdn.seq_table([0, 5, 70, 200])
    p.workspace_bytes = lib.gdn_fwd_varlen_workspace_bytes(ctypes.byref(p), cu)
    assert lib.gdn_fwd_varlen(ctypes.byref(p), None, None) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_fwd_varlen(ctypes.byref(p), gdn.seq_table([0, 5, 4, 200]), None) == gdn.GDN_ERR_INVALID_ARG
    small = fake_params(lib, B=3, T=1, H=2, D=64)
    small.workspace_bytes = p.workspace_bytes - 1
    assert lib.gdn_fwd_varlen(ctypes.byref(small), cu, None) == gdn.GDN_ERR_WORKSPACE
    q = fake_params(lib, B=3, T=1, H=2, D=64)
    q.workspace_bytes = p.workspace_bytes
    q.o = q.q + 256  # output over an input
    assert lib.gdn_fwd_varlen(ctypes.byref(q), cu, None) == gdn.GDN_ERR_INVALID_ARG
    q = fake_params(lib, B=3, T=1, H=2, D=64)
    q.Dk = q.Dv = 96
    q.workspace_bytes = 1 << 30
    assert lib.gdn_fwd_varlen(ctypes.byref(q), cu, None) == gdn.GDN_ERR_UNSUPPORTED


# ---- the backward pass

def fake_bwd(lib, B=2, T=300, H=3, D=128, io=gdn.GDN_BF16):
    p = gdn.GdnBwdParams()
    p.B, p.T, p.H, p.Dk, p.Dv, p.io_dtype = B, T, H, D, D, io
    base, step = 1 << 44, 1 << 36
    names = [f[0] for f in gdn.GdnBwdParams._fields_ if f[1] is ctypes.c_void_p]
    for i, nm in enumerate(names):
        setattr(p, nm, base + i * step)
    p.eps_l2 = p.eps_norm = 1e-6
    p.workspace_bytes = lib.gdn_bwd_workspace_bytes(ctypes.byref(p))
    assert p.workspace_bytes > 0
    return p


def test_bwd_workspace_bytes(lib):
    p = fake_bwd(lib, B=1, T=32760, H=12, D=128)
    NC, D = 512, 128
    per_chunk = (909 * D + 12416 + 2 * D * D) * 4
    sink = 12 * D * D * 4  # the chains' stores past either end
    assert abs(p.workspace_bytes - 12 * NC * per_chunk - sink) <= 4 * 256
    q = gdn.GdnBwdParams()
    q.B, q.T, q.H, q.Dk, q.Dv, q.io_dtype = 1, 100, 2, 96, 96, gdn.GDN_BF16
    assert lib.gdn_bwd_workspace_bytes(ctypes.byref(q)) == 0
    assert lib.gdn_bwd_workspace_bytes(None) == 0


def test_bwd_launch_names(lib):
    n = lib.gdn_bwd_launch_count()
    assert n == 7
    names = gdn.gdn_bwd_launch_names()
    assert names[0] == "bwd_prep_kernel" and names[-1] == "bwd_reduce_kernel" and len(set(names)) == n
    assert lib.gdn_bwd_launch_name(n) is None and lib.gdn_bwd_launch_name(-1) is None


BWD_CASES = [
    ("dy NULL", lambda p: setattr(p, "dy", None), gdn.GDN_ERR_INVALID_ARG),
    ("dq NULL", lambda p: setattr(p, "dq", None), gdn.GDN_ERR_INVALID_ARG),
    ("dconv_v NULL", lambda p: setattr(p, "dconv_v", None), gdn.GDN_ERR_INVALID_ARG),
    ("eps_norm < 0", lambda p: setattr(p, "eps_norm", -1.0), gdn.GDN_ERR_INVALID_ARG),
    ("eps_l2 inf", lambda p: setattr(p, "eps_l2", float("inf")), gdn.GDN_ERR_INVALID_ARG),
    ("B = 0", lambda p: setattr(p, "B", 0), gdn.GDN_ERR_INVALID_ARG),
    ("io dtype 7", lambda p: setattr(p, "io_dtype", 7), gdn.GDN_ERR_INVALID_ARG),
    ("Dk != Dv", lambda p: setattr(p, "Dv", 64), gdn.GDN_ERR_UNSUPPORTED),
    ("D = 32", lambda p: (setattr(p, "Dk", 32), setattr(p, "Dv", 32)), gdn.GDN_ERR_UNSUPPORTED),
    ("dq misaligned", lambda p: setattr(p, "dq", p.dq + 1), gdn.GDN_ERR_ALIGNMENT),
    ("dlog_a misaligned", lambda p: setattr(p, "dlog_a", p.dlog_a + 2), gdn.GDN_ERR_ALIGNMENT),
    ("k not 16-byte aligned", lambda p: setattr(p, "k", p.k + 8), gdn.GDN_ERR_ALIGNMENT),
    ("conv_v not 16-byte aligned", lambda p: setattr(p, "conv_v", p.conv_v + 4), gdn.GDN_ERR_ALIGNMENT),
    ("workspace NULL", lambda p: setattr(p, "workspace", None), gdn.GDN_ERR_WORKSPACE),
    ("workspace too small", lambda p: setattr(p, "workspace_bytes", p.workspace_bytes - 1), gdn.GDN_ERR_WORKSPACE),
    ("workspace misaligned", lambda p: setattr(p, "workspace", p.workspace + 16), gdn.GDN_ERR_ALIGNMENT),
    ("dk overlaps k", lambda p: setattr(p, "dk", p.k + 512), gdn.GDN_ERR_INVALID_ARG),
    ("dgate overlaps dq", lambda p: setattr(p, "dgate", p.dq + 512), gdn.GDN_ERR_INVALID_ARG),
    ("dS0 overlaps the workspace", lambda p: setattr(p, "dS0", p.workspace + 4096), gdn.GDN_ERR_INVALID_ARG),
    ("dnorm_w overlaps dS_T", lambda p: setattr(p, "dnorm_w", p.dS_T), gdn.GDN_ERR_INVALID_ARG),
    ("reverse = 2", lambda p: setattr(p, "reverse", 2), gdn.GDN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,mutate,expect", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_validation_errors(lib, name, mutate, expect):
    p = fake_bwd(lib)
    mutate(p)
    assert lib.gdn_bwd(ctypes.byref(p), None) == expect, name


def test_bwd_optional_outputs_may_be_null(lib):
    # with the optional pointers NULL the call still fails only on the fake workspace size
    p = fake_bwd(lib)
    p.dnorm_w = p.dS0 = p.norm_w = p.S0 = p.dS_T = None
    p.workspace_bytes -= 1
    assert lib.gdn_bwd(ctypes.byref(p), None) == gdn.GDN_ERR_WORKSPACE


def test_bwd_timed_needs_events(lib):
    p = fake_bwd(lib)
    n = 2 * lib.gdn_bwd_launch_count()
    events = (ctypes.c_void_p * (n - 1))()
    assert lib.gdn_bwd_timed(ctypes.byref(p), events, n - 1, None) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_bwd_timed(ctypes.byref(p), None, n, None) == gdn.GDN_ERR_INVALID_ARG


def test_bwd_varlen_table_checks(lib):
    p = fake_bwd(lib, B=3, T=150)
    p.T = 0  # ignored by the varlen calls
    IP = ctypes.c_int * 4
    assert lib.gdn_bwd_varlen_workspace_bytes(ctypes.byref(p), IP(0, 100, 250, 300)) > 0
    assert lib.gdn_bwd_varlen_workspace_bytes(ctypes.byref(p), IP(1, 100, 250, 300)) == 0   # not from 0
    assert lib.gdn_bwd_varlen_workspace_bytes(ctypes.byref(p), IP(0, 100, 100, 300)) == 0   # an empty sequence
    # the longest sequence (150 tokens) sets the chunk records: the same bytes as a B = 3, T = 150 batch,
    # plus the table
    q = fake_bwd(lib, B=3, T=150)
    assert lib.gdn_bwd_varlen_workspace_bytes(ctypes.byref(p), IP(0, 100, 250, 300)) == q.workspace_bytes + 256
    assert lib.gdn_bwd_varlen(ctypes.byref(p), IP(0, 100, 90, 300), None) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_bwd_varlen(ctypes.byref(p), None, None) == gdn.GDN_ERR_INVALID_ARG



def test_noalloc_refuses_sizes_beyond_its_array(lib):
    """gdn_fwd_noalloc's workspace is a fixed 64 MiB device array: larger
    sizes are refused before any device call (so this runs without a GPU)."""
    p = fake_params(lib, B=1, T=32760, H=12, D=128)
    assert lib.gdn_fwd_workspace_bytes(ctypes.byref(p)) > (64 << 20)
    assert lib.gdn_fwd_noalloc(ctypes.byref(p), None) == gdn.GDN_ERR_WORKSPACE
    p.T = 0
    assert lib.gdn_fwd_noalloc(ctypes.byref(p), None) == gdn.GDN_ERR_INVALID_ARG

// gdn_proj.hip -- host side of the token mixer entry points declared in
// include/gdn.h: the projections (gdn_in_proj, gdn_out_proj) and the whole
// mixer (gdn_mixer_fwd): validation, workspace carve-up and the launches.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/gdn.h"
#include "gemm.hpp"
#include "internal.hpp"

namespace {

using gdn::bf16;

struct Span {
    uintptr_t lo, hi;
};
Span span(const void *p, size_t bytes) { return Span{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr double kMaxElems = 2147483647.0;  // 32-bit element offsets inside the kernel

// outputs must not overlap any input or each other
template <size_t NI, size_t NO>
bool disjoint(const Span (&ins)[NI], const Span (&outs)[NO]) {
    for (size_t o = 0; o < NO; ++o) {
        for (size_t i = 0; i < NI; ++i)
            if (overlap(outs[o], ins[i])) return false;
        for (size_t j = o + 1; j < NO; ++j)
            if (overlap(outs[o], outs[j])) return false;
    }
    return true;
}

gdn_status set_gemm_attributes() {
    static std::once_flag once;
    static gdn_status result = GDN_OK;
    std::call_once(once, [] {
        const void *fns[] = {reinterpret_cast<const void *>(&gdn::gdn_gemm_kernel<gdn::kEpiPlain>),
                             reinterpret_cast<const void *>(&gdn::gdn_gemm_kernel<gdn::kEpiInProj>)};
        for (const void *fn : fns)
            if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, gdn::gemm::LDS_BYTES) !=
                hipSuccess)
                result = GDN_ERR_HIP;
    });
    return result;
}

// The launch of one GEMM (tile counts filled in), for a stream or a plan.
template <int EPI>
gdn_status gemm_launch_desc(gdn::GemmArgs &a, gdn_internal::ExtLaunch &e) {
    a.mt = (a.M + gdn::gemm::BM - 1) / gdn::gemm::BM;
    a.nt = (a.N + gdn::gemm::BN - 1) / gdn::gemm::BN;
    const long long tiles = (long long)a.mt * a.nt;
    const long long grid = (tiles + 7) / 8 * 8;  // a multiple of 8 for the XCD placement
    if (grid > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;
    static_assert(sizeof(gdn::GemmArgs) <= sizeof(e.args), "GEMM arguments fit a plan launch");
    e = gdn_internal::ExtLaunch{};
    e.fn = reinterpret_cast<const void *>(&gdn::gdn_gemm_kernel<EPI>);
    e.grid = dim3((unsigned)grid);
    e.block = dim3(gdn::gemm::THREADS);
    e.smem = gdn::gemm::LDS_BYTES;
    memcpy(e.args, &a, sizeof(a));
    e.name = EPI == gdn::kEpiInProj ? "gdn_gemm_kernel<in-projection>" : "gdn_gemm_kernel<plain>";
    return GDN_OK;
}

template <int EPI>
gdn_status launch_gemm(gdn::GemmArgs &a, hipStream_t s) {
    gdn_status st = set_gemm_attributes();
    if (st != GDN_OK) return st;
    gdn_internal::ExtLaunch e;
    st = gemm_launch_desc<EPI>(a, e);
    if (st != GDN_OK) return st;
    void *kargs[] = {e.args};
    if (hipLaunchKernel(e.fn, e.grid, e.block, kargs, e.smem, s) != hipSuccess) return GDN_ERR_HIP;
    return GDN_OK;
}

gdn_status in_proj_check(const gdn_in_proj_params *p) {
    if (!p || p->B < 1 || p->T < 1 || p->H < 1 || p->D < 1 || p->C < 1) return GDN_ERR_INVALID_ARG;
    if (!p->x || !p->w_in || !p->A_log || !p->q || !p->k || !p->v || !p->gate || !p->beta || !p->log_a)
        return GDN_ERR_INVALID_ARG;
    const double M = (double)p->B * p->T, HD = (double)p->H * p->D, N = 4 * HD + 2.0 * p->H;
    if (p->C % 64 != 0 || (long long)HD % 16 != 0 || M * p->C > kMaxElems || N * p->C > kMaxElems ||
        M * HD > kMaxElems)
        return GDN_ERR_UNSUPPORTED;
    const void *al16[] = {p->x, p->w_in, p->b_in, p->q, p->k, p->v, p->gate};
    for (const void *ptr : al16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_ALIGNMENT;
    const void *al4[] = {p->A_log, p->beta, p->log_a};
    for (const void *ptr : al4)
        if (!aligned(ptr, 4)) return GDN_ERR_ALIGNMENT;
    const size_t m = (size_t)M, hd = (size_t)HD, n = (size_t)N, c = p->C, h = p->H;
    const Span ins[] = {span(p->x, m * c * 2), span(p->w_in, n * c * 2), span(p->b_in, p->b_in ? n * 4 : 0),
                        span(p->A_log, h * 4)};
    const Span outs[] = {span(p->q, m * hd * 2),    span(p->k, m * hd * 2),    span(p->v, m * hd * 2),
                         span(p->gate, m * hd * 2), span(p->beta, m * h * 4), span(p->log_a, m * h * 4)};
    if (!disjoint(ins, outs)) return GDN_ERR_INVALID_ARG;
    return GDN_OK;
}

// The in-projection of token rows [row0, row0 + rows) of the B T rows.
gdn::GemmArgs in_proj_args(const gdn_in_proj_params *p, size_t row0, int rows) {
    gdn::GemmArgs a = {};
    const size_t HD = (size_t)p->H * p->D;
    a.M = rows; a.N = 4 * p->H * p->D + 2 * p->H; a.K = p->C;
    a.x = static_cast<const bf16 *>(p->x) + row0 * p->C;
    a.w = static_cast<const bf16 *>(p->w_in);
    a.bias = p->b_in;
    a.dst[0] = static_cast<bf16 *>(p->q) + row0 * HD;
    a.dst[1] = static_cast<bf16 *>(p->k) + row0 * HD;
    a.dst[2] = static_cast<bf16 *>(p->v) + row0 * HD;
    a.dst[3] = static_cast<bf16 *>(p->gate) + row0 * HD;
    a.HD = p->H * p->D; a.H = p->H;
    a.beta = p->beta + row0 * p->H; a.log_a = p->log_a + row0 * p->H; a.A_log = p->A_log;
    return a;
}

gdn_status in_proj_launch(const gdn_in_proj_params *p, hipStream_t s) {
    gdn::GemmArgs a = in_proj_args(p, 0, p->B * p->T);
    return launch_gemm<gdn::kEpiInProj>(a, s);
}

gdn_status out_proj_check(const gdn_out_proj_params *p) {
    if (!p || p->B < 1 || p->T < 1 || p->H < 1 || p->D < 1 || p->C < 1) return GDN_ERR_INVALID_ARG;
    if (!p->y || !p->w_out || !p->out) return GDN_ERR_INVALID_ARG;
    const double M = (double)p->B * p->T, HD = (double)p->H * p->D;
    if ((long long)HD % 64 != 0 || p->C % 8 != 0 || M * HD > kMaxElems || (double)p->C * HD > kMaxElems ||
        M * p->C > 4.0e12)
        return GDN_ERR_UNSUPPORTED;
    const void *al16[] = {p->y, p->w_out, p->b_out, p->out};
    for (const void *ptr : al16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_ALIGNMENT;
    const size_t m = (size_t)M, hd = (size_t)HD, c = p->C;
    const Span ins[] = {span(p->y, m * hd * 2), span(p->w_out, c * hd * 2), span(p->b_out, p->b_out ? c * 4 : 0)};
    const Span outs[] = {span(p->out, m * c * 2)};
    if (!disjoint(ins, outs)) return GDN_ERR_INVALID_ARG;
    return GDN_OK;
}

// The out-projection of token rows [row0, row0 + rows) of the B T rows.
gdn::GemmArgs out_proj_args(const gdn_out_proj_params *p, size_t row0, int rows) {
    gdn::GemmArgs a = {};
    a.M = rows; a.N = p->C; a.K = p->H * p->D;
    a.x = static_cast<const bf16 *>(p->y) + row0 * ((size_t)p->H * p->D);
    a.w = static_cast<const bf16 *>(p->w_out);
    a.bias = p->b_out;
    a.out = static_cast<bf16 *>(p->out) + row0 * p->C;
    return a;
}

gdn_status out_proj_launch(const gdn_out_proj_params *p, hipStream_t s) {
    gdn::GemmArgs a = out_proj_args(p, 0, p->B * p->T);
    return launch_gemm<gdn::kEpiPlain>(a, s);
}

// ------------------------------------------------------------------ mixer
constexpr size_t kWsAlign = 256;
size_t round_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct MixerParts {
    gdn_in_proj_params in;
    gdn_fwd_params layer;
    gdn_out_proj_params out;
    size_t total;  // workspace bytes
};

// The three stages' params with the intermediates carved from the workspace
// (q, k, v, gate, y as [B, T, H, D] bf16, b and log a as [B, T, H] fp32, then
// the layer's own workspace).  sizes_only: leave every pointer NULL.
bool mixer_parts(const gdn_mixer_params *p, MixerParts &mp, bool sizes_only) {
    if (!p || p->B < 1 || p->T < 1 || p->H < 1 || p->D < 1 || p->C < 1) return false;
    const size_t m = (size_t)p->B * p->T, hd = (size_t)p->H * p->D, h = p->H;
    if ((double)m * hd > 4.0e12) return false;
    mp = MixerParts{};
    gdn_fwd_params &L = mp.layer;
    L.B = p->B; L.T = p->T; L.H = p->H; L.Dk = p->D; L.Dv = p->D; L.io_dtype = GDN_BF16;
    const size_t layer_ws = gdn_fwd_workspace_bytes(&L);
    if (layer_ws == 0) return false;
    size_t off[8], o = 0;
    for (int i = 0; i < 5; ++i) { off[i] = o; o += round_up(m * hd * 2); }   // q k v gate y
    for (int i = 5; i < 7; ++i) { off[i] = o; o += round_up(m * h * 4); }    // b, log a
    off[7] = o;
    mp.total = o + layer_ws;
    char *ws = sizes_only ? nullptr : static_cast<char *>(p->workspace);
    auto at = [&](int i) -> void * { return ws ? ws + off[i] : nullptr; };

    gdn_in_proj_params &I = mp.in;
    I.B = p->B; I.T = p->T; I.H = p->H; I.D = p->D; I.C = p->C;
    I.x = p->x; I.w_in = p->w_in; I.b_in = p->b_in; I.A_log = p->A_log;
    I.q = at(0); I.k = at(1); I.v = at(2); I.gate = at(3);
    I.beta = static_cast<float *>(at(5)); I.log_a = static_cast<float *>(at(6));

    L.q = at(0); L.k = at(1); L.v = at(2); L.gate = at(3);
    L.beta = static_cast<const float *>(at(5)); L.log_a = static_cast<const float *>(at(6));
    L.conv_q = p->conv_q; L.conv_k = p->conv_k; L.conv_v = p->conv_v;
    L.norm_w = p->norm_w; L.eps_l2 = p->eps_l2; L.eps_norm = p->eps_norm;
    L.S0 = p->S0; L.S_T = p->S_T; L.o = at(4); L.reverse = 0;
    L.workspace = at(7); L.workspace_bytes = ws ? p->workspace_bytes - off[7] : 0;

    gdn_out_proj_params &O = mp.out;
    O.B = p->B; O.T = p->T; O.H = p->H; O.D = p->D; O.C = p->C;
    O.y = at(4); O.w_out = p->w_out; O.b_out = p->b_out; O.out = p->out;
    return true;
}

// The mixer: the in-projection over all rows on the caller's stream, then the
// layer with the out-projection woven into its launch plan, split by the
// layer's chunk ranges and batch rows: the out-projection of range i runs on
// a library stream after the output kernel of range i, beside the chain's
// later ranges.  Each output element is computed by the same products in the
// same order as by one out-projection over all rows, so the result is the
// same.  (Measured at T = 32760, C = 1536, H = 12, d = 128: 1.36 -> 1.30 ms.
// The in-projection split the same way, ahead of each range's prep, made the
// call slower, 1.62 ms: its workgroups hold whole CUs, 144 KB of LDS each,
// and delay the chain.)
gdn_status mixer_staged(const MixerParts &mp, hipStream_t s) {
    gdn_status st = in_proj_launch(&mp.in, s);
    if (st != GDN_OK) return st;
    std::vector<int> bounds;
    gdn_internal::scan_range_bounds(&mp.layer, bounds);
    const int R = (int)bounds.size() - 1, T = mp.layer.T;
    std::vector<std::vector<gdn_internal::ExtLaunch>> post(R);
    for (int i = 0; i < R; ++i) {
        const int t0 = bounds[i] * 64, t1 = std::min(bounds[i + 1] * 64, T);
        for (int b = 0; b < mp.layer.B; ++b) {
            gdn_internal::ExtLaunch e;
            gdn::GemmArgs ao = out_proj_args(&mp.out, (size_t)b * T + t0, t1 - t0);
            st = gemm_launch_desc<gdn::kEpiPlain>(ao, e);
            if (st != GDN_OK) return st;
            post[i].push_back(e);
        }
    }
    return gdn_internal::fwd_call_staged(&mp.layer, post, s);
}

gdn_status mixer_call(const gdn_mixer_params *p, hipEvent_t *timing, int n_timing, hipStream_t s) {
    MixerParts mp;
    if (!mixer_parts(p, mp, true)) return GDN_ERR_INVALID_ARG;
    if (!p->workspace || p->workspace_bytes < mp.total) return GDN_ERR_WORKSPACE;
    if (!aligned(p->workspace, kWsAlign)) return GDN_ERR_ALIGNMENT;
    mixer_parts(p, mp, false);
    // the caller's buffers must not overlap the workspace
    const size_t m = (size_t)p->B * p->T, hd = (size_t)p->H * p->D, n = 4 * hd + 2 * p->H, c = p->C;
    const Span ws[] = {span(p->workspace, mp.total)};
    const size_t hh = p->H, dd = p->D;
    const Span user[] = {span(p->x, m * c * 2),          span(p->w_in, n * c * 2),
                         span(p->w_out, c * hd * 2),     span(p->out, m * c * 2),
                         span(p->b_in, p->b_in ? n * 4 : 0), span(p->b_out, p->b_out ? c * 4 : 0),
                         span(p->A_log, hh * 4),         span(p->conv_q, hd * 16),
                         span(p->conv_k, hd * 16),       span(p->conv_v, hd * 16),
                         span(p->norm_w, p->norm_w ? hd * 4 : 0),
                         span(p->S0, p->S0 ? (size_t)p->B * hh * dd * dd * 4 : 0),
                         span(p->S_T, p->S_T ? (size_t)p->B * hh * dd * dd * 4 : 0)};
    if (!disjoint(user, ws)) return GDN_ERR_INVALID_ARG;
    // the mixer's outputs must not overlap any of its inputs or each other
    const Span ins[] = {user[0], user[1], user[2], user[4], user[5], user[6], user[7], user[8], user[9], user[10],
                        user[11]};
    const Span outs[] = {user[3], user[12]};
    if (!disjoint(ins, outs)) return GDN_ERR_INVALID_ARG;
    // every check of the three stages before the first launch
    gdn_status st = in_proj_check(&mp.in);
    if (st == GDN_OK) st = gdn_internal::fwd_check(&mp.layer);
    if (st == GDN_OK) st = out_proj_check(&mp.out);
    if (st != GDN_OK) return st;
    if (!timing) return mixer_staged(mp, s);
    int n_layer = gdn_fwd_launch_count(&mp.layer, 0);
    if (n_layer < 0 || n_timing < 4 + 2 * n_layer) return GDN_ERR_INVALID_ARG;
    auto rec = [&](int i) { return !timing || hipEventRecord(timing[i], s) == hipSuccess; };
    if (!rec(0)) return GDN_ERR_HIP;
    st = in_proj_launch(&mp.in, s);
    if (st != GDN_OK) return st;
    if (!rec(1)) return GDN_ERR_HIP;
    st = gdn_internal::fwd_call(&mp.layer, timing ? timing + 4 : nullptr, timing ? n_timing - 4 : 0, s);
    if (st != GDN_OK) return st;
    if (!rec(2)) return GDN_ERR_HIP;
    st = out_proj_launch(&mp.out, s);
    if (st != GDN_OK) return st;
    if (!rec(3)) return GDN_ERR_HIP;
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_in_proj(const gdn_in_proj_params *p, struct ihipStream_t *stream) {
    try {
        gdn_status st = in_proj_check(p);
        return st != GDN_OK ? st : in_proj_launch(p, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

gdn_status gdn_out_proj(const gdn_out_proj_params *p, struct ihipStream_t *stream) {
    try {
        gdn_status st = out_proj_check(p);
        return st != GDN_OK ? st : out_proj_launch(p, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

size_t gdn_mixer_workspace_bytes(const gdn_mixer_params *p) {
    try {
        MixerParts mp;
        return mixer_parts(p, mp, true) ? mp.total : 0;
    } catch (...) {
        return 0;
    }
}

gdn_status gdn_mixer_fwd(const gdn_mixer_params *p, struct ihipStream_t *stream) {
    try {
        return mixer_call(p, nullptr, 0, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

gdn_status gdn_mixer_fwd_timed(const gdn_mixer_params *p, struct ihipEvent_t **events, int n_events,
                               struct ihipStream_t *stream) {
    if (!events) return GDN_ERR_INVALID_ARG;
    try {
        return mixer_call(p, reinterpret_cast<hipEvent_t *>(events), n_events, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

}  // extern "C"

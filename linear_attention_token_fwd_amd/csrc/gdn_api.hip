// gdn_api.hip -- host side of the C ABI declared in include/gdn.h:
// argument validation, workspace carve-up and the launch sequence.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/gdn.h"
#include "kernels.hpp"

namespace {

using gdn::bf16;

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t rec, gC, ows, total;  // byte offsets (total = size)
};

int n_chunks(int T) { return (T + gdn::kChunk - 1) / gdn::kChunk; }

size_t elem_size(gdn_dtype d) { return d == GDN_BF16 ? 2 : 4; }

// scans = number of scans whose partial outputs are alive at once (1 or 2)
Layout layout(const gdn_fwd_params *p, int scans) {
    const size_t B = p->B, H = p->H, D = p->Dk, NC = n_chunks(p->T);
    Layout L;
    size_t off = 0;
    L.rec = off;
    off += round_up(B * H * NC * 320 * D * elem_size(p->io_dtype));
    L.gC = off;
    off += round_up(B * H * NC * sizeof(float));
    L.ows = off;
    off += scans * round_up(B * H * NC * 64 * D * sizeof(float));
    L.total = off;
    return L;
}

bool sizes_ok(const gdn_fwd_params *p) {
    if (!p) return false;
    if (p->B < 1 || p->T < 1 || p->H < 1 || p->Dk < 1 || p->Dv < 1) return false;
    if (p->io_dtype != GDN_F32 && p->io_dtype != GDN_BF16) return false;
    // element counts must fit the 32-bit grid and the index arithmetic below
    const double elems = (double)p->B * p->T * p->H * (double)(p->Dk > p->Dv ? p->Dk : p->Dv);
    if (elems > 4.0e12) return false;
    if ((double)p->B * p->H > 65535.0 * 65535.0 || p->H > 65535 || p->B > 65535) return false;
    return true;
}

bool supported(const gdn_fwd_params *p) {
    if (p->Dk != p->Dv) return false;
    if (p->io_dtype == GDN_BF16) return p->Dk == 64 || p->Dk == 128;
    return p->Dk == 64;
}

struct Range {
    uintptr_t lo, hi;
};
Range rng(const void *ptr, size_t bytes) { return Range{(uintptr_t)ptr, (uintptr_t)ptr + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

gdn_status validate(const gdn_fwd_params *p, const float *S_T_rev, int scans) {
    if (!sizes_ok(p)) return GDN_ERR_INVALID_ARG;
    if (!p->q || !p->k || !p->v || !p->log_a || !p->beta || !p->gate || !p->conv_q || !p->conv_k ||
        !p->conv_v || !p->o)
        return GDN_ERR_INVALID_ARG;
    if (!(std::isfinite(p->eps_l2) && p->eps_l2 >= 0.f && std::isfinite(p->eps_norm) && p->eps_norm >= 0.f))
        return GDN_ERR_INVALID_ARG;
    if (p->reverse != 0 && p->reverse != 1) return GDN_ERR_INVALID_ARG;
    if (!supported(p)) return GDN_ERR_UNSUPPORTED;
    const size_t es = elem_size(p->io_dtype);
    const size_t B = p->B, T = p->T, H = p->H, D = p->Dk;
    const size_t tok = B * T * H;
    const void *vec16[] = {p->q, p->k, p->v, p->gate, p->o, p->conv_q, p->conv_k, p->conv_v,
                           p->S0, p->S_T, S_T_rev};
    for (const void *ptr : vec16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_ALIGNMENT;
    const void *vec4[] = {p->log_a, p->beta, p->norm_w};
    for (const void *ptr : vec4)
        if (ptr && !aligned(ptr, 4)) return GDN_ERR_ALIGNMENT;
    const Layout L = layout(p, scans);
    if (!p->workspace || p->workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
    if (!aligned(p->workspace, kAlign)) return GDN_ERR_ALIGNMENT;
    // outputs must not overlap any input, the workspace or each other
    const Range ins[] = {rng(p->q, tok * D * es),          rng(p->k, tok * D * es),
                         rng(p->v, tok * D * es),          rng(p->gate, tok * D * es),
                         rng(p->log_a, tok * 4),           rng(p->beta, tok * 4),
                         rng(p->conv_q, H * D * 16),       rng(p->conv_k, H * D * 16),
                         rng(p->conv_v, H * D * 16),       rng(p->norm_w, p->norm_w ? H * D * 4 : 0),
                         rng(p->S0, p->S0 ? B * H * D * D * 4 : 0)};
    const Range ws = rng(p->workspace, L.total);
    const Range outs[] = {rng(p->o, tok * D * es), rng(p->S_T, p->S_T ? B * H * D * D * 4 : 0),
                          rng(S_T_rev, S_T_rev ? B * H * D * D * 4 : 0)};
    for (const Range &o : outs) {
        for (const Range &i : ins)
            if (overlap(o, i)) return GDN_ERR_INVALID_ARG;
        if (overlap(o, ws)) return GDN_ERR_INVALID_ARG;
    }
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return GDN_ERR_INVALID_ARG;
    for (const Range &i : ins)
        if (overlap(ws, i)) return GDN_ERR_INVALID_ARG;
    return GDN_OK;
}

// A call is a short fixed sequence of kernel launches on one stream.
struct Launch {
    const void *fn;
    dim3 grid, block;
    size_t smem;
    unsigned char args[256];
};

struct Plan {
    Launch l[8];
    int n = 0;
    template <class Args> void add(const void *fn, dim3 grid, dim3 block, size_t smem, const Args &a) {
        static_assert(sizeof(Args) <= sizeof(Launch::args), "kernel arguments too large");
        Launch &L = l[n++];
        L.fn = fn; L.grid = grid; L.block = block; L.smem = smem;
        memcpy(L.args, &a, sizeof(Args));
    }
    // events: NULL, or n + 1 events recorded before each launch and after the last
    gdn_status run(hipStream_t s, hipEvent_t *events) const {
        for (int i = 0; i < n; ++i) {
            if (events && hipEventRecord(events[i], s) != hipSuccess) return GDN_ERR_HIP;
            void *kargs[] = {const_cast<unsigned char *>(l[i].args)};
            if (hipLaunchKernel(l[i].fn, l[i].grid, l[i].block, kargs, l[i].smem, s) != hipSuccess)
                return GDN_ERR_HIP;
        }
        if (events && hipEventRecord(events[n], s) != hipSuccess) return GDN_ERR_HIP;
        return GDN_OK;
    }
};

// One scan: prep + state.  ows receives that scan's unnormalised output.
template <class T, int D>
gdn_status plan_scan(Plan &plan, const gdn_fwd_params *p, int reverse, const float *S0, float *S_T, float *ows,
                     char *ws, const Layout &L) {
    const int NC = n_chunks(p->T);
    gdn::PrepArgs pa;
    pa.B = p->B; pa.T = p->T; pa.H = p->H; pa.NC = NC; pa.reverse = reverse;
    pa.q = p->q; pa.k = p->k; pa.v = p->v;
    pa.log_a = p->log_a; pa.beta = p->beta;
    pa.conv_q = p->conv_q; pa.conv_k = p->conv_k; pa.conv_v = p->conv_v;
    pa.eps_l2 = p->eps_l2;
    pa.rec = ws + L.rec;
    pa.gC = reinterpret_cast<float *>(ws + L.gC);
    const size_t smem = sizeof(gdn::PrepSmem<T, D>);
    const void *prep = reinterpret_cast<const void *>(&gdn::gdn_prep_kernel<T, D>);
    if (hipFuncSetAttribute(prep, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
        return GDN_ERR_HIP;
    plan.add(prep, dim3(NC, p->H, p->B), dim3(gdn::kThreads), smem, pa);
    gdn::StateArgs sa;
    sa.B = p->B; sa.T = p->T; sa.H = p->H; sa.NC = NC;
    sa.rec = ws + L.rec;
    sa.gC = reinterpret_cast<const float *>(ws + L.gC);
    sa.S0 = S0; sa.S_T = S_T; sa.ows = ows;
    const int used = p->B * p->H * (D / 16);
    plan.add(reinterpret_cast<const void *>(&gdn::gdn_state_kernel<T, D>), dim3((used + 7) / 8 * 8),
             dim3(gdn::kThreads), 0, sa);
    return GDN_OK;
}

template <class T, int D>
void plan_norm(Plan &plan, const gdn_fwd_params *p, int reverse, const float *ows, const float *ows2) {
    gdn::NormArgs na;
    na.B = p->B; na.T = p->T; na.H = p->H; na.NC = n_chunks(p->T); na.reverse = reverse;
    na.ows = ows; na.ows2 = ows2;
    na.gate = p->gate; na.norm_w = p->norm_w; na.eps = p->eps_norm; na.out = p->o;
    constexpr int tok_per_block = gdn::kThreads / (D / 8);
    plan.add(reinterpret_cast<const void *>(&gdn::gdn_norm_kernel<T, D>),
             dim3((p->T + tok_per_block - 1) / tok_per_block, p->H, p->B), dim3(gdn::kThreads), 0, na);
}

template <class T, int D>
gdn_status plan_fwd(Plan &plan, const gdn_fwd_params *p, const float *S_T_rev, bool bidir) {
    const Layout L = layout(p, bidir ? 2 : 1);
    char *ws = static_cast<char *>(p->workspace);
    float *ows = reinterpret_cast<float *>(ws + L.ows);
    const size_t ows_bytes = round_up((size_t)p->B * p->H * n_chunks(p->T) * 64 * D * sizeof(float));
    gdn_status st = plan_scan<T, D>(plan, p, bidir ? 0 : p->reverse, p->S0, p->S_T, ows, ws, L);
    if (st != GDN_OK) return st;
    if (!bidir) {
        plan_norm<T, D>(plan, p, p->reverse, ows, nullptr);
        return GDN_OK;
    }
    float *ows2 = reinterpret_cast<float *>(ws + L.ows + ows_bytes);
    st = plan_scan<T, D>(plan, p, 1, p->S0, const_cast<float *>(S_T_rev), ows2, ws, L);
    if (st != GDN_OK) return st;
    plan_norm<T, D>(plan, p, 0, ows, ows2);
    return GDN_OK;
}

gdn_status make_plan(Plan &plan, const gdn_fwd_params *p, const float *S_T_rev, bool bidir) {
    if (p->io_dtype == GDN_BF16 && p->Dk == 128) return plan_fwd<bf16, 128>(plan, p, S_T_rev, bidir);
    if (p->io_dtype == GDN_BF16 && p->Dk == 64) return plan_fwd<bf16, 64>(plan, p, S_T_rev, bidir);
    if (p->io_dtype == GDN_F32 && p->Dk == 64) return plan_fwd<float, 64>(plan, p, S_T_rev, bidir);
    return GDN_ERR_UNSUPPORTED;
}

gdn_status call(const gdn_fwd_params *p, const float *S_T_rev, bool bidir, hipEvent_t *events, int n_events,
                hipStream_t s) {
    gdn_status st = validate(p, S_T_rev, bidir ? 2 : 1);
    if (st != GDN_OK) return st;
    if (bidir && p->reverse != 0) return GDN_ERR_INVALID_ARG;
    Plan plan;
    st = make_plan(plan, p, S_T_rev, bidir);
    if (st != GDN_OK) return st;
    if (events && n_events < plan.n + 1) return GDN_ERR_INVALID_ARG;
    return plan.run(s, events);
}

}  // namespace

extern "C" {

size_t gdn_fwd_workspace_bytes(const gdn_fwd_params *p) {
    if (!sizes_ok(p)) return 0;
    return layout(p, 1).total;
}

size_t gdn_fwd_bidir_workspace_bytes(const gdn_fwd_params *p) {
    if (!sizes_ok(p)) return 0;
    return layout(p, 2).total;
}

gdn_status gdn_fwd(const gdn_fwd_params *p, struct ihipStream_t *stream) {
    try {
        return call(p, nullptr, false, nullptr, 0, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

gdn_status gdn_fwd_bidir(const gdn_fwd_params *p, float *S_T_rev, struct ihipStream_t *stream) {
    try {
        return call(p, S_T_rev, true, nullptr, 0, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

int gdn_fwd_launch_count(const gdn_fwd_params *p, int bidirectional) {
    if (!sizes_ok(p) || !supported(p)) return -1;
    return bidirectional ? 5 : 3;
}

gdn_status gdn_fwd_timed(const gdn_fwd_params *p, float *S_T_rev, int bidirectional, struct ihipEvent_t **events,
                         int n_events, struct ihipStream_t *stream) {
    if (!events) return GDN_ERR_INVALID_ARG;
    try {
        return call(p, S_T_rev, bidirectional != 0, reinterpret_cast<hipEvent_t *>(events), n_events, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

const char *gdn_fwd_launch_name(const gdn_fwd_params *p, int bidirectional, int i) {
    static const char *uni[] = {"gdn_prep_kernel", "gdn_state_kernel", "gdn_norm_kernel"};
    static const char *bi[] = {"gdn_prep_kernel", "gdn_state_kernel", "gdn_prep_kernel", "gdn_state_kernel",
                               "gdn_norm_kernel"};
    const int n = gdn_fwd_launch_count(p, bidirectional);
    if (i < 0 || i >= n) return nullptr;
    return bidirectional ? bi[i] : uni[i];
}

const char *gdn_status_string(gdn_status s) {
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case GDN_ERR_ALIGNMENT: return "misaligned pointer";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP runtime or launch failure";
    }
    return "unknown status";
}

}  // extern "C"

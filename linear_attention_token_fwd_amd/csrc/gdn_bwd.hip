// gdn_bwd.hip -- host side of gdn_bwd (include/gdn.h): argument checks,
// workspace carve-up and the seven launches of the backward pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>

#include "../../include/gdn.h"
#include "bwd.hpp"
#include "internal.hpp"

namespace {

using gdn::bf16;
using gdnb::NT;

constexpr size_t kAlign = 256;
constexpr int kLaunches = 7;
const char *const kNames[kLaunches] = {"bwd_prep_kernel", "bwd_state_kernel",    "bwd_out_kernel",   "bwd_dstate_kernel",
                                       "bwd_grad_kernel", "bwd_prologue_kernel", "bwd_reduce_kernel"};

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int n_chunks(int T) { return (T + gdnb::C - 1) / gdnb::C; }
size_t elem_size(gdn_dtype d) { return d == GDN_BF16 ? 2 : 4; }

size_t rec_floats(int D) { return D == 128 ? gdnb::Rec<128>::SIZE : gdnb::Rec<64>::SIZE; }

struct Layout {
    size_t rec, part_conv, part_norm, sink, seq, total;
};

// varlen: room for the device copy of a sequence table of B + 1 ints
Layout layout(const gdn_bwd_params *p, bool varlen = false) {
    const size_t B = p->B, H = p->H, D = p->Dk, NC = n_chunks(p->T);
    Layout L;
    L.rec = 0;
    L.part_conv = round_up(B * H * NC * rec_floats(p->Dk) * sizeof(float));
    L.part_norm = L.part_conv + round_up(B * NC * H * 12 * D * sizeof(float));
    L.sink = L.part_norm + round_up(B * NC * H * D * sizeof(float));
    L.seq = L.sink + round_up(B * H * D * D * sizeof(float));
    L.total = L.seq + (varlen ? round_up((B + 1) * sizeof(int)) : 0);
    return L;
}

bool sizes_ok(const gdn_bwd_params *p) {
    if (!p) return false;
    if (p->B < 1 || p->T < 1 || p->H < 1 || p->Dk < 1 || p->Dv < 1) return false;
    const int dt = gdn_internal::dtype_code(p->io_dtype);
    if (dt != GDN_F32 && dt != GDN_BF16) return false;
    if (p->H > 65535 || p->B > 65535) return false;
    // element counts inside one launch's index arithmetic, and the chunk grid
    if ((double)p->B * p->T * p->H * (double)p->Dk > 4.0e12) return false;
    if (n_chunks(p->T) > 1 << 30) return false;
    return true;
}

struct Span {
    uintptr_t lo, hi;
};
Span span(const void *ptr, size_t bytes) { return Span{(uintptr_t)ptr, (uintptr_t)ptr + bytes}; }
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// rows: token rows of the per-token tensors (B T, or the packed total)
gdn_status validate(const gdn_bwd_params *p, size_t rows, bool varlen) {
    if (!sizes_ok(p)) return GDN_ERR_INVALID_ARG;
    if (p->Dk != p->Dv) return GDN_ERR_UNSUPPORTED;
    if (p->Dk != 64 && p->Dk != 128) return GDN_ERR_UNSUPPORTED;
    if (!p->q || !p->k || !p->v || !p->log_a || !p->beta || !p->gate || !p->conv_q || !p->conv_k || !p->conv_v ||
        !p->dy || !p->dq || !p->dk || !p->dv || !p->dgate || !p->dlog_a || !p->dbeta || !p->dconv_q ||
        !p->dconv_k || !p->dconv_v)
        return GDN_ERR_INVALID_ARG;
    if (!(p->eps_l2 >= 0.f) || !(p->eps_norm >= 0.f) || !std::isfinite(p->eps_l2) || !std::isfinite(p->eps_norm))
        return GDN_ERR_INVALID_ARG;
    if (p->reverse != 0 && p->reverse != 1) return GDN_ERR_INVALID_ARG;
    const size_t B = p->B, H = p->H, D = p->Dk, es = elem_size(p->io_dtype);
    const size_t tok = rows * H * D * es, gates = rows * H * 4, conv = H * D * 16, st = B * H * D * D * 4;
    const Span in[] = {span(p->q, tok),      span(p->k, tok),      span(p->v, tok),
                       span(p->gate, tok),   span(p->dy, tok),     span(p->log_a, gates),
                       span(p->beta, gates), span(p->conv_q, conv), span(p->conv_k, conv),
                       span(p->conv_v, conv), span(p->norm_w, p->norm_w ? H * D * 4 : 0),
                       span(p->S0, p->S0 ? st : 0), span(p->dS_T, p->dS_T ? st : 0)};
    const Span out[] = {span(p->dq, tok),          span(p->dk, tok),          span(p->dv, tok),
                        span(p->dgate, tok),       span(p->dlog_a, gates),    span(p->dbeta, gates),
                        span(p->dconv_q, conv),    span(p->dconv_k, conv),    span(p->dconv_v, conv),
                        span(p->dnorm_w, p->dnorm_w ? H * D * 4 : 0), span(p->dS0, p->dS0 ? st : 0),
                        span(p->workspace, p->workspace ? p->workspace_bytes : 0)};
    const int nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Span &s : in)
            if (overlap(out[i], s)) return GDN_ERR_INVALID_ARG;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return GDN_ERR_INVALID_ARG;
    }
    // q, k, v and the conv weights are read with 16-byte loads; every other
    // tensor is accessed element by element
    const void *vec[] = {p->q, p->k, p->v, p->conv_q, p->conv_k, p->conv_v};
    for (const void *ptr : vec)
        if (!aligned(ptr, 16)) return GDN_ERR_ALIGNMENT;
    const void *io[] = {p->gate, p->dy, p->dq, p->dk, p->dv, p->dgate};
    for (const void *ptr : io)
        if (!aligned(ptr, es)) return GDN_ERR_ALIGNMENT;
    const void *f32[] = {p->log_a, p->beta, p->norm_w, p->S0, p->dS_T, p->dlog_a, p->dbeta, p->dconv_q,
                         p->dconv_k, p->dconv_v, p->dnorm_w, p->dS0};
    for (const void *ptr : f32)
        if (ptr && !aligned(ptr, 4)) return GDN_ERR_ALIGNMENT;
    if (!p->workspace || p->workspace_bytes < layout(p, varlen).total) return GDN_ERR_WORKSPACE;
    if (!aligned(p->workspace, kAlign)) return GDN_ERR_ALIGNMENT;
    return GDN_OK;
}

template <int D> size_t prep_lds() { return (3 * 64 * (D + 4) + 2 * 64 * 68 + 3 * 64 + 4 * 16 * 20) * sizeof(float); }
template <int D> size_t prologue_lds() {
    typedef gdnb::PrologueCfg<D> P;
    return ((64 + 3) * P::LZ + P::RUNS * D * 4) * sizeof(float);
}
template <int D> size_t grad_lds() { return (3 * 64 * (D + 4) + 3 * 64 * 68 + 11 * 64) * sizeof(float); }

gdn_status set_attributes() {
    static std::once_flag once;
    static gdn_status result = GDN_OK;
    std::call_once(once, [] {
        struct A {
            const void *fn;
            size_t lds;
        } attrs[] = {
            {reinterpret_cast<const void *>(&gdnb::bwd_prep_kernel<bf16, 128>), prep_lds<128>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_prep_kernel<bf16, 64>), prep_lds<64>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_prep_kernel<float, 128>), prep_lds<128>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_prep_kernel<float, 64>), prep_lds<64>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_prologue_kernel<bf16, 128>), prologue_lds<128>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_prologue_kernel<bf16, 64>), prologue_lds<64>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_prologue_kernel<float, 128>), prologue_lds<128>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_prologue_kernel<float, 64>), prologue_lds<64>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_grad_kernel<128>), grad_lds<128>()},
            {reinterpret_cast<const void *>(&gdnb::bwd_grad_kernel<64>), grad_lds<64>()},
        };
        for (const A &a : attrs)
            if (hipFuncSetAttribute(a.fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)a.lds) != hipSuccess)
                result = GDN_ERR_HIP;
    });
    return result;
}

// Per device: one library stream (default priority, non-blocking) and the
// events of the fork and joins, created on first use and kept.
constexpr int kMaxRanges = 8;
struct DeviceRes {
    hipStream_t side = nullptr;
    hipEvent_t ev[2 * kMaxRanges + 4] = {};
};
std::mutex g_mutex;
std::map<int, DeviceRes> g_res;

gdn_status device_res(DeviceRes *&out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    auto it = g_res.find(dev);
    if (it == g_res.end()) {
        DeviceRes r;
        if (hipStreamCreateWithFlags(&r.side, hipStreamNonBlocking) != hipSuccess) return GDN_ERR_HIP;
        for (hipEvent_t &e : r.ev)
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return GDN_ERR_HIP;
        it = g_res.emplace(dev, r).first;
    }
    out = &it->second;
    return GDN_OK;
}

template <class IO, int D> gdnb::Args make_args(const gdn_bwd_params *p, const int *cu_dev) {
    const Layout L = layout(p, cu_dev != nullptr);
    gdnb::Args a;
    a.B = p->B, a.T = p->T, a.H = p->H, a.NC = n_chunks(p->T), a.c0 = 0, a.c1 = a.NC;
    a.q = p->q, a.k = p->k, a.v = p->v, a.gate = p->gate, a.dy = p->dy;
    a.log_a = p->log_a, a.beta = p->beta;
    a.conv_q = p->conv_q, a.conv_k = p->conv_k, a.conv_v = p->conv_v, a.norm_w = p->norm_w;
    a.S0 = p->S0, a.dS_T = p->dS_T;
    a.eps_l2 = p->eps_l2, a.eps_norm = p->eps_norm;
    a.dq = p->dq, a.dk = p->dk, a.dv = p->dv, a.dgate = p->dgate;
    a.dlog_a = p->dlog_a, a.dbeta = p->dbeta;
    a.dconv_q = p->dconv_q, a.dconv_k = p->dconv_k, a.dconv_v = p->dconv_v;
    a.dnorm_w = p->dnorm_w, a.dS0 = p->dS0;
    a.rec = gdn_internal::at_offset<float>(p->workspace, L.rec);
    a.part_conv = gdn_internal::at_offset<float>(p->workspace, L.part_conv);
    a.part_norm = gdn_internal::at_offset<float>(p->workspace, L.part_norm);
    a.sink = gdn_internal::at_offset<float>(p->workspace, L.sink);
    a.reverse = p->reverse;
    a.cu = cu_dev;
    return a;
}

// Launch i of the call on stream s over chunks [c0, c1) (per-chunk kernels
// and chains; the last two kernels always cover everything).
template <class IO, int D> bool launch(int i, gdnb::Args a, int c0, int c1, hipStream_t s) {
    using namespace gdnb;
    a.c0 = c0, a.c1 = c1;
    const dim3 chunks(c1 - c0, a.H, a.B);
    // chains: 8 equal slices of the work list (whole heads each), one per XCD
    const dim3 rows(8 * ((a.B * a.H + 7) / 8) * (D / 16));
    switch (i) {
    case 0: bwd_prep_kernel<IO, D><<<chunks, GNT, prep_lds<D>(), s>>>(a); break;
    case 1: bwd_state_kernel<D><<<rows, NT, 0, s>>>(a); break;
    case 2: bwd_out_kernel<IO, D><<<chunks, NT, 0, s>>>(a); break;
    case 3: bwd_dstate_kernel<D><<<rows, NT, 0, s>>>(a); break;
    case 4: bwd_grad_kernel<D><<<chunks, GNT, grad_lds<D>(), s>>>(a); break;
    case 5: bwd_prologue_kernel<IO, D><<<chunks, NT, prologue_lds<D>(), s>>>(a); break;
    default: bwd_reduce_kernel<D><<<dim3((a.H * D * 13 + 63) / 64), NT, 0, s>>>(a); break;
    }
    return hipGetLastError() == hipSuccess;
}

// Timed: every kernel once over all chunks on the caller's stream, events
// around each.
template <class IO, int D> gdn_status launch_timed(const gdn_bwd_params *p, hipEvent_t *ev, hipStream_t s) {
    const gdnb::Args a = make_args<IO, D>(p, nullptr);
    for (int i = 0; i < kLaunches; ++i) {
        (void)hipEventRecord(ev[2 * i], s);
        if (!launch<IO, D>(i, a, 0, a.NC, s)) return GDN_ERR_HIP;
        (void)hipEventRecord(ev[2 * i + 1], s);
    }
    return GDN_OK;
}

// The call: the two chains run over ranges of about 64 chunks on the
// caller's stream; the output backward of a range follows its forward-chain
// range, and the gradient kernel of a range its reverse-chain range, on the
// library stream, so that both use the CUs the chains leave idle.
template <class IO, int D> gdn_status launch_all(const gdn_bwd_params *p, const int *cu_dev, hipStream_t s) {
    const gdnb::Args a = make_args<IO, D>(p, cu_dev);
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceRes *res = nullptr;
    gdn_status st = device_res(res);
    if (st != GDN_OK) return st;
    const int NC = a.NC, R = std::min(kMaxRanges, std::max(1, (NC + 63) / 64));
    int bound[kMaxRanges + 1];
    for (int r = 0; r <= R; ++r) bound[r] = (int)((long long)NC * r / R);
    hipStream_t side = res->side;
    hipEvent_t *ev = res->ev;
    int e = 0;
    auto fork = [&](hipStream_t from, hipStream_t to) {
        hipEvent_t x = ev[e++];
        return hipEventRecord(x, from) == hipSuccess && hipStreamWaitEvent(to, x, 0) == hipSuccess;
    };
    if (!fork(s, side)) return GDN_ERR_HIP;
    if (!launch<IO, D>(0, a, 0, NC, s)) return GDN_ERR_HIP;
    for (int r = 0; r < R; ++r) {
        if (!launch<IO, D>(1, a, bound[r], bound[r + 1], s) || !fork(s, side) ||
            !launch<IO, D>(2, a, bound[r], bound[r + 1], side))
            return GDN_ERR_HIP;
    }
    if (!fork(side, s)) return GDN_ERR_HIP;
    for (int r = R - 1; r >= 0; --r) {
        if (!launch<IO, D>(3, a, bound[r], bound[r + 1], s) || !fork(s, side) ||
            !launch<IO, D>(4, a, bound[r], bound[r + 1], side))
            return GDN_ERR_HIP;
    }
    if (!fork(side, s)) return GDN_ERR_HIP;
    if (!launch<IO, D>(5, a, 0, NC, s) || !launch<IO, D>(6, a, 0, NC, s)) return GDN_ERR_HIP;
    return GDN_OK;
}

gdn_status call(const gdn_bwd_params *p, hipEvent_t *ev, int n_ev, hipStream_t s) {
    if (!sizes_ok(p)) return GDN_ERR_INVALID_ARG;
    gdn_status st = validate(p, (size_t)p->B * p->T, false);
    if (st != GDN_OK) return st;
    if (ev && n_ev < 2 * kLaunches) return GDN_ERR_INVALID_ARG;
    st = set_attributes();
    if (st != GDN_OK) return st;
    if (ev) {
        if (p->io_dtype == GDN_BF16)
            return p->Dk == 128 ? launch_timed<bf16, 128>(p, ev, s) : launch_timed<bf16, 64>(p, ev, s);
        return p->Dk == 128 ? launch_timed<float, 128>(p, ev, s) : launch_timed<float, 64>(p, ev, s);
    }
    if (p->io_dtype == GDN_BF16)
        return p->Dk == 128 ? launch_all<bf16, 128>(p, nullptr, s) : launch_all<bf16, 64>(p, nullptr, s);
    return p->Dk == 128 ? launch_all<float, 128>(p, nullptr, s) : launch_all<float, 64>(p, nullptr, s);
}

// Variable-length batch: the params with T = the longest length, or an error
// for a malformed table (cu[0] = 0, every length >= 1).
gdn_status varlen_params(const gdn_bwd_params *p, const int *cu, gdn_bwd_params &q) {
    if (!p || !cu || p->B < 1) return GDN_ERR_INVALID_ARG;
    if (cu[0] != 0) return GDN_ERR_INVALID_ARG;
    int longest = 0;
    for (int b = 0; b < p->B; ++b) {
        const long long len = (long long)cu[b + 1] - cu[b];
        if (len < 1) return GDN_ERR_INVALID_ARG;
        if (len > longest) longest = (int)len;
    }
    q = *p;
    q.T = longest;
    return GDN_OK;
}

gdn_status varlen_call(const gdn_bwd_params *p, const int *cu, hipStream_t s) {
    gdn_bwd_params q;
    gdn_status st = varlen_params(p, cu, q);
    if (st != GDN_OK) return st;
    if (!sizes_ok(&q)) return GDN_ERR_INVALID_ARG;
    st = validate(&q, (size_t)cu[q.B], true);
    if (st != GDN_OK) return st;
    st = set_attributes();
    if (st != GDN_OK) return st;
    int *cu_dev = gdn_internal::at_offset<int>(q.workspace, layout(&q, true).seq);
    // the table goes to the workspace first, on the caller's stream
    if (hipMemcpyAsync(cu_dev, cu, sizeof(int) * (q.B + 1), hipMemcpyHostToDevice, s) != hipSuccess)
        return GDN_ERR_HIP;
    if (q.io_dtype == GDN_BF16)
        return q.Dk == 128 ? launch_all<bf16, 128>(&q, cu_dev, s) : launch_all<bf16, 64>(&q, cu_dev, s);
    return q.Dk == 128 ? launch_all<float, 128>(&q, cu_dev, s) : launch_all<float, 64>(&q, cu_dev, s);
}

}  // namespace

extern "C" {

size_t gdn_bwd_workspace_bytes(const gdn_bwd_params *p) {
    if (!sizes_ok(p) || p->Dk != p->Dv || (p->Dk != 64 && p->Dk != 128)) return 0;
    return layout(p).total;
}

gdn_status gdn_bwd(const gdn_bwd_params *p, struct ihipStream_t *stream) {
    try {
        return call(p, nullptr, 0, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

gdn_status gdn_bwd_timed(const gdn_bwd_params *p, struct ihipEvent_t **events, int n_events,
                         struct ihipStream_t *stream) {
    if (!events) return GDN_ERR_INVALID_ARG;
    try {
        return call(p, events, n_events, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

size_t gdn_bwd_varlen_workspace_bytes(const gdn_bwd_params *p, const int *cu_seqlens) {
    gdn_bwd_params q;
    if (varlen_params(p, cu_seqlens, q) != GDN_OK) return 0;
    if (!sizes_ok(&q) || q.Dk != q.Dv || (q.Dk != 64 && q.Dk != 128)) return 0;
    return layout(&q, true).total;
}

gdn_status gdn_bwd_varlen(const gdn_bwd_params *p, const int *cu_seqlens, struct ihipStream_t *stream) {
    try {
        return varlen_call(p, cu_seqlens, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

int gdn_bwd_launch_count(void) { return kLaunches; }

const char *gdn_bwd_launch_name(int i) { return i >= 0 && i < kLaunches ? kNames[i] : nullptr; }

}  // extern "C"

// gdn_proj.hip -- host side of the token mixer projections declared in
// include/gdn.h (gdn_in_proj, gdn_out_proj): validation and the launch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/gdn.h"
#include "gemm.hpp"

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

template <int EPI>
gdn_status launch_gemm(gdn::GemmArgs &a, hipStream_t s) {
    gdn_status st = set_gemm_attributes();
    if (st != GDN_OK) return st;
    a.mt = (a.M + gdn::gemm::BM - 1) / gdn::gemm::BM;
    a.nt = (a.N + gdn::gemm::BN - 1) / gdn::gemm::BN;
    const long long tiles = (long long)a.mt * a.nt;
    const long long grid = (tiles + 7) / 8 * 8;  // a multiple of 8 for the XCD placement
    if (grid > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;
    void *kargs[] = {&a};
    if (hipLaunchKernel(reinterpret_cast<const void *>(&gdn::gdn_gemm_kernel<EPI>), dim3((unsigned)grid),
                        dim3(gdn::gemm::THREADS), kargs, gdn::gemm::LDS_BYTES, s) != hipSuccess)
        return GDN_ERR_HIP;
    return GDN_OK;
}

gdn_status in_proj(const gdn_in_proj_params *p, hipStream_t s) {
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

    gdn::GemmArgs a = {};
    a.M = (int)M; a.N = (int)N; a.K = p->C;
    a.x = static_cast<const bf16 *>(p->x);
    a.w = static_cast<const bf16 *>(p->w_in);
    a.bias = p->b_in;
    a.dst[0] = static_cast<bf16 *>(p->q);
    a.dst[1] = static_cast<bf16 *>(p->k);
    a.dst[2] = static_cast<bf16 *>(p->v);
    a.dst[3] = static_cast<bf16 *>(p->gate);
    a.HD = (int)HD; a.H = p->H;
    a.beta = p->beta; a.log_a = p->log_a; a.A_log = p->A_log;
    return launch_gemm<gdn::kEpiInProj>(a, s);
}

gdn_status out_proj(const gdn_out_proj_params *p, hipStream_t s) {
    if (!p || p->B < 1 || p->T < 1 || p->H < 1 || p->D < 1 || p->C < 1) return GDN_ERR_INVALID_ARG;
    if (!p->y || !p->w_out || !p->out) return GDN_ERR_INVALID_ARG;
    const double M = (double)p->B * p->T, HD = (double)p->H * p->D;
    if ((long long)HD % 64 != 0 || p->C % 4 != 0 || M * HD > kMaxElems || (double)p->C * HD > kMaxElems ||
        M * p->C > 4.0e12)
        return GDN_ERR_UNSUPPORTED;
    const void *al16[] = {p->y, p->w_out, p->b_out, p->out};
    for (const void *ptr : al16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_ALIGNMENT;
    const size_t m = (size_t)M, hd = (size_t)HD, c = p->C;
    const Span ins[] = {span(p->y, m * hd * 2), span(p->w_out, c * hd * 2), span(p->b_out, p->b_out ? c * 4 : 0)};
    const Span outs[] = {span(p->out, m * c * 2)};
    if (!disjoint(ins, outs)) return GDN_ERR_INVALID_ARG;

    gdn::GemmArgs a = {};
    a.M = (int)M; a.N = p->C; a.K = (int)HD;
    a.x = static_cast<const bf16 *>(p->y);
    a.w = static_cast<const bf16 *>(p->w_out);
    a.bias = p->b_out;
    a.out = static_cast<bf16 *>(p->out);
    return launch_gemm<gdn::kEpiPlain>(a, s);
}

}  // namespace

extern "C" {

gdn_status gdn_in_proj(const gdn_in_proj_params *p, struct ihipStream_t *stream) {
    try {
        return in_proj(p, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

gdn_status gdn_out_proj(const gdn_out_proj_params *p, struct ihipStream_t *stream) {
    try {
        return out_proj(p, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

}  // extern "C"

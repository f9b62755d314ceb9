// gdn_api.hip -- host side of the C ABI declared in include/gdn.h:
// argument validation, workspace carve-up and the launch sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/gdn.h"
#include "internal.hpp"
#include "kernels.hpp"

namespace {

using gdn::bf16;

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    // per scan: chunk records, e^{g_C}, chunk-entry states, two state hand-off buffers;
    // then, for two scans, one fp32 accumulator for the sum of their outputs
    // then, for variable-length batches, the device copy of the sequence table
    size_t rec, gC, sc, smid, per_scan, acc, seq, total;  // byte offsets within a scan's block, sizes
};

int n_chunks(int T) { return (T + gdn::kChunk - 1) / gdn::kChunk; }

size_t elem_size(gdn_dtype d) { return d == GDN_BF16 ? 2 : 4; }

// scans = number of scans whose buffers are alive at once (1 or 2); varlen:
// room for a sequence table of B + 1 ints
Layout layout(const gdn_fwd_params *p, int scans, bool varlen = false) {
    const size_t B = p->B, T = p->T, H = p->H, D = p->Dk, NC = n_chunks(p->T), es = elem_size(p->io_dtype);
    Layout L;
    size_t off = 0;
    L.rec = off;
    off += round_up(B * H * NC * 320 * D * es);
    L.gC = off;
    off += round_up(B * H * NC * sizeof(float));
    L.sc = off;
    off += round_up(B * H * NC * 16 * D * es * (D / 16));
    L.smid = off;
    off += 2 * round_up(B * H * D * D * sizeof(float));
    L.per_scan = off;
    L.acc = scans * off;
    L.seq = L.acc + (scans == 2 ? round_up(B * T * H * D * sizeof(float)) : 0);
    L.total = L.seq + (varlen ? round_up((B + 1) * sizeof(int)) : 0);
    return L;
}

bool sizes_ok(const gdn_fwd_params *p) {
    if (!p) return false;
    if (p->B < 1 || p->T < 1 || p->H < 1 || p->Dk < 1 || p->Dv < 1) return false;
    const int dt = gdn_internal::dtype_code(p->io_dtype);
    if (dt != GDN_F32 && dt != GDN_BF16) return false;
    // element counts must fit the 32-bit grid and the index arithmetic below
    const double elems = (double)p->B * p->T * p->H * (double)(p->Dk > p->Dv ? p->Dk : p->Dv);
    if (elems > 4.0e12) return false;
    if ((double)p->B * p->H > 65535.0 * 65535.0 || p->H > 65535 || p->B > 65535) return false;
    return true;
}

bool supported(const gdn_fwd_params *p) {
    return p->Dk == p->Dv && (p->Dk == 64 || p->Dk == 128);
}

struct Range {
    uintptr_t lo, hi;
};
Range rng(const void *ptr, size_t bytes) { return Range{(uintptr_t)ptr, (uintptr_t)ptr + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// tokens: rows of the per-token tensors (B T, or the packed total of a
// variable-length batch, which also needs the sequence table's room)
gdn_status validate(const gdn_fwd_params *p, const float *S_T_rev, int scans, size_t tokens, bool varlen) {
    if (!sizes_ok(p)) return GDN_ERR_INVALID_ARG;
    if (!p->q || !p->k || !p->v || !p->log_a || !p->beta || !p->gate || !p->conv_q || !p->conv_k ||
        !p->conv_v || !p->o)
        return GDN_ERR_INVALID_ARG;
    if (!(std::isfinite(p->eps_l2) && p->eps_l2 >= 0.f && std::isfinite(p->eps_norm) && p->eps_norm >= 0.f))
        return GDN_ERR_INVALID_ARG;
    if (p->reverse != 0 && p->reverse != 1) return GDN_ERR_INVALID_ARG;
    if (!supported(p)) return GDN_ERR_UNSUPPORTED;
    const size_t es = elem_size(p->io_dtype);
    const size_t B = p->B, H = p->H, D = p->Dk;
    const size_t tok = tokens * H;
    const void *vec16[] = {p->q, p->k, p->v, p->gate, p->o, p->conv_q, p->conv_k, p->conv_v,
                           p->S0, p->S_T, S_T_rev};
    for (const void *ptr : vec16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_ALIGNMENT;
    const void *vec4[] = {p->log_a, p->beta, p->norm_w};
    for (const void *ptr : vec4)
        if (ptr && !aligned(ptr, 4)) return GDN_ERR_ALIGNMENT;
    const Layout L = layout(p, scans, varlen);
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

// A call is a fixed plan of kernel launches spread over up to four streams:
// stream 0 is the caller's, streams 1-3 belong to the library (one set per
// device, created on first use, default priority).  (A process gets four
// hardware queues by default, so more streams would only share them.)  Events order the streams:
// every library stream first waits for the caller's stream at the start of
// the call, and the caller's stream finally waits for every library stream,
// so the call behaves as one stream-ordered operation on the caller's stream.
constexpr int kStreams = 4;

struct Launch {
    const void *fn;
    dim3 grid, block;
    size_t smem;
    unsigned char args[160];
    const char *name;
};

struct Op {
    enum Kind { LAUNCH, RECORD, WAIT } kind;
    int stream;
    int event;  // plan-local event index for RECORD / WAIT, launch index for LAUNCH
};

struct Plan {
    std::vector<Op> ops;
    std::vector<Launch> launches;
    int n_events = 0;
    template <class Args>
    void launch(int stream, const char *name, const void *fn, dim3 grid, dim3 block, size_t smem, const Args &a) {
        static_assert(sizeof(Args) <= sizeof(Launch::args), "kernel arguments too large");
        Launch L = {};  // zero-filled: the argument bytes past sizeof(Args) take part in plan_key()
        L.fn = fn; L.grid = grid; L.block = block; L.smem = smem; L.name = name;
        memcpy(L.args, &a, sizeof(Args));
        ops.push_back(Op{Op::LAUNCH, stream, (int)launches.size()});
        launches.push_back(L);
    }
    void launch_ext(int stream, const gdn_internal::ExtLaunch &e) {
        Launch L = {};
        L.fn = e.fn; L.grid = e.grid; L.block = e.block; L.smem = e.smem; L.name = e.name;
        static_assert(sizeof(e.args) == sizeof(L.args), "argument buffers");
        memcpy(L.args, e.args, sizeof(L.args));
        ops.push_back(Op{Op::LAUNCH, stream, (int)launches.size()});
        launches.push_back(L);
    }
    int record(int stream) {
        ops.push_back(Op{Op::RECORD, stream, n_events});
        return n_events++;
    }
    void wait(int stream, int event) { ops.push_back(Op{Op::WAIT, stream, event}); }
};

struct DeviceRes {
    hipStream_t streams[kStreams] = {};
    std::vector<hipEvent_t> events;
};

std::mutex g_mutex;
std::map<int, DeviceRes> g_res;

// Caller holds g_mutex.
gdn_status device_res(int n_events, DeviceRes *&out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    DeviceRes &r = g_res[dev];
    for (int i = 1; i < kStreams; ++i)
        if (!r.streams[i] && hipStreamCreateWithFlags(&r.streams[i], hipStreamNonBlocking) != hipSuccess)
            return GDN_ERR_HIP;
    while ((int)r.events.size() < n_events) {
        hipEvent_t e;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return GDN_ERR_HIP;
        r.events.push_back(e);
    }
    out = &r;
    return GDN_OK;
}

// Enqueue the plan's operations (caller holds g_mutex).  timing: NULL, or 2
// events per launch recorded right before and right after it.
gdn_status enqueue_ops(const Plan &plan, const hipStream_t *streams, DeviceRes *r, hipEvent_t *timing) {
    for (const Op &op : plan.ops) {
        hipStream_t s = streams[op.stream];
        if (op.kind == Op::RECORD) {
            if (hipEventRecord(r->events[op.event], s) != hipSuccess) return GDN_ERR_HIP;
        } else if (op.kind == Op::WAIT) {
            if (hipStreamWaitEvent(s, r->events[op.event], 0) != hipSuccess) return GDN_ERR_HIP;
        } else {
            const Launch &L = plan.launches[op.event];
            if (timing && hipEventRecord(timing[2 * op.event], s) != hipSuccess) return GDN_ERR_HIP;
            void *kargs[] = {const_cast<unsigned char *>(L.args)};
            if (hipLaunchKernel(L.fn, L.grid, L.block, kargs, L.smem, s) != hipSuccess) return GDN_ERR_HIP;
            if (timing && hipEventRecord(timing[2 * op.event + 1], s) != hipSuccess) return GDN_ERR_HIP;
        }
    }
    return GDN_OK;
}

// Graphs.  A plan can be recorded once as a HIP graph (capturing the caller's
// stream, which forks onto the library streams through the plan's events and
// joins back) and replayed for identical plans: one graph launch in place of
// dozens of launches and event operations, which removes the gaps between
// dependent kernels on different streams (measured 5-9% faster per call on
// the single-scan workloads; the bidirectional plan runs faster directly).
// Plans are identical when their operations and every launch's kernel, shape
// and argument bytes (pointers included) are.  A plan is recorded the second
// time it is seen (the first call runs directly), so callers whose buffers
// move from call to call never pay for recording.  The most recently used
// g_graph_limit graphs are kept per process (0: no graphs, every plan runs
// directly), and the keys of the last kSeenPlans plans seen once.
constexpr int kMaxCachedGraphs = 64;
constexpr size_t kSeenPlans = 16;
size_t g_graph_limit = 8;  // guarded by g_mutex, like the lists below
struct CachedGraph {
    int device;
    std::vector<unsigned char> key;
    hipGraphExec_t exec;
};
std::vector<CachedGraph> g_graphs;  // least recently used first
std::vector<std::pair<int, std::vector<unsigned char>>> g_seen;  // oldest first

// Caller holds g_mutex.  Destroys the least recently used graphs until at
// most `keep` remain.
void evict_graphs(size_t keep) {
    while (g_graphs.size() > keep) {
        (void)hipGraphExecDestroy(g_graphs.front().exec);
        g_graphs.erase(g_graphs.begin());
    }
}

std::vector<unsigned char> plan_key(const Plan &plan) {
    std::vector<unsigned char> k;
    auto put = [&](const void *p, size_t n) {
        const unsigned char *b = static_cast<const unsigned char *>(p);
        k.insert(k.end(), b, b + n);
    };
    for (const Op &op : plan.ops) {
        const int v[3] = {(int)op.kind, op.stream, op.event};
        put(v, sizeof(v));
    }
    for (const Launch &L : plan.launches) {
        const unsigned g[6] = {L.grid.x, L.grid.y, L.grid.z, L.block.x, L.block.y, L.block.z};
        put(&L.fn, sizeof(L.fn));
        put(g, sizeof(g));
        put(&L.smem, sizeof(L.smem));
        put(L.args, sizeof(L.args));
    }
    return k;
}

// Caller holds g_mutex.  Replays the cached graph of this plan, or records,
// caches and launches one; returns false (nothing enqueued) when a graph
// cannot be used, and the plan then runs directly.
bool launch_as_graph(const Plan &plan, const hipStream_t *streams, DeviceRes *r, gdn_status &st) {
    hipStream_t caller = streams[0];
    if (g_graph_limit == 0) return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (caller == nullptr || hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return false;  // the null stream cannot be captured; the caller's own capture records the plan itself
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::vector<unsigned char> key = plan_key(plan);
    for (size_t i = 0; i < g_graphs.size(); ++i) {
        if (g_graphs[i].device != dev || g_graphs[i].key != key) continue;
        CachedGraph hit = std::move(g_graphs[i]);
        g_graphs.erase(g_graphs.begin() + i);
        g_graphs.push_back(std::move(hit));
        st = hipGraphLaunch(g_graphs.back().exec, caller) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
        return true;
    }
    bool seen = false;
    for (size_t i = 0; i < g_seen.size() && !seen; ++i) {
        if (g_seen[i].first != dev || g_seen[i].second != key) continue;
        g_seen.erase(g_seen.begin() + i);
        seen = true;
    }
    if (!seen) {  // first sighting: remember it and run directly
        if (g_seen.size() >= kSeenPlans) g_seen.erase(g_seen.begin());
        g_seen.emplace_back(dev, std::move(key));
        return false;
    }
    if (hipStreamBeginCapture(caller, hipStreamCaptureModeThreadLocal) != hipSuccess) return false;
    const gdn_status recorded = enqueue_ops(plan, streams, r, nullptr);
    hipGraph_t graph = nullptr;
    const hipError_t ended = hipStreamEndCapture(caller, &graph);
    hipGraphExec_t exec = nullptr;
    const bool ok = recorded == GDN_OK && ended == hipSuccess && graph &&
                    hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess;
    if (graph) (void)hipGraphDestroy(graph);
    if (!ok) return false;
    evict_graphs(g_graph_limit - 1);
    g_graphs.push_back(CachedGraph{dev, std::move(key), exec});
    st = hipGraphLaunch(exec, caller) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    return true;
}

// timing: NULL, or 2 events per launch recorded right before and right after
// it (timed plans always run directly).  as_graph: replay the plan as a
// cached graph where possible.
gdn_status run_plan(const Plan &plan, hipStream_t caller, hipEvent_t *timing, bool as_graph = false) {
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceRes *r = nullptr;
    gdn_status st = device_res(plan.n_events, r);
    if (st != GDN_OK) return st;
    hipStream_t streams[kStreams];
    streams[0] = caller;
    for (int i = 1; i < kStreams; ++i) streams[i] = r->streams[i];
    if (as_graph && !timing && launch_as_graph(plan, streams, r, st)) return st;
    return enqueue_ops(plan, streams, r, timing);
}

// Chunk ranges of a scan: R = ceil(NC / target) ranges of equal size, at
// most 16 unless a range would exceed the state kernel's limit.  Each chain
// launch pays for filling its operand registers and for the hand-over of the
// state, and the first prep range and the last output range run alone.
// Measured (MI355X, H = 12, d = 128), one scan with the launch graph
// replayed: T = 32760 (512 chunks) 4 ranges of 128 0.622 ms, 3 of 171 0.625,
// 2 of 256 0.633; T = 75600 (1182 chunks) ranges of 128 1.367-1.374 ms, of
// 169 1.344-1.352, of 197 1.384; T = 27280 with H = 24: 4 or 3 ranges 0.804.
// Both scans co-scheduled (launched directly), T = 126360 (1975 chunks):
// ranges of 123 4.60 ms, 165 4.45, 200 4.35, 247 4.30, 330 4.25, 395 4.25.
constexpr int kRangeTarget = 170;       // one scan
constexpr int kRangeTargetBidir = 400;  // both scans co-scheduled
int n_ranges(int NC, int target = kRangeTarget) {
    int R = (NC + target - 1) / target;
    R = R < 1 ? 1 : (R > 16 ? 16 : R);
    const int need = (NC + gdn::kStateMaxRange - 1) / gdn::kStateMaxRange;
    return R < need ? need : R;
}
int range_begin(int NC, int R, int i) { return (int)((long long)NC * i / R); }

// Dynamic LDS of the state kernel: none.  Its ~20 KB of static LDS lets a
// prep or output workgroup share its CU, so a range's state launch starts
// without waiting for CUs to drain (measured faster overall than keeping the
// chain alone on its CUs).
constexpr size_t kStateReserveLds = 0;
template <class T, int D> constexpr size_t state_lds() {
    return kStateReserveLds;
}

struct ScanBufs {
    char *rec, *sc;
    float *gC, *smid[2];
};

ScanBufs scan_bufs(const gdn_fwd_params *p, const Layout &L, int scan) {
    char *base = gdn_internal::at_offset(p->workspace, (size_t)scan * L.per_scan);
    ScanBufs b;
    b.rec = gdn_internal::at_offset(base, L.rec);
    b.sc = gdn_internal::at_offset(base, L.sc);
    b.gC = gdn_internal::at_offset<float>(base, L.gC);
    const size_t sbytes = round_up((size_t)p->B * p->H * p->Dk * p->Dk * sizeof(float));
    b.smid[0] = gdn_internal::at_offset<float>(base, L.smid);
    b.smid[1] = gdn_internal::at_offset<float>(base, L.smid + sbytes);
    return b;
}

template <class T, int D>
gdn::PrepArgs prep_args(const gdn_fwd_params *p, int reverse, const ScanBufs &sb, int c_begin, const int *cu) {
    gdn::PrepArgs pa;
    memset(&pa, 0, sizeof(pa));  // padding too: the argument bytes key the graph cache
    pa.B = p->B; pa.T = p->T; pa.H = p->H; pa.NC = n_chunks(p->T); pa.reverse = reverse;
    pa.cu = cu;
    pa.c_begin = c_begin;
    pa.q = p->q; pa.k = p->k; pa.v = p->v;
    pa.log_a = p->log_a; pa.beta = p->beta;
    pa.conv_q = p->conv_q; pa.conv_k = p->conv_k; pa.conv_v = p->conv_v;
    pa.eps_l2 = p->eps_l2;
    pa.rec = sb.rec;
    pa.gC = sb.gC;
    return pa;
}

template <class T, int D>
gdn::StateArgs state_args(const gdn_fwd_params *p, const ScanBufs &sb, int c0, int c1, const float *S_in,
                          float *S_out, float *S_T, const int *cu) {
    gdn::StateArgs sa;
    memset(&sa, 0, sizeof(sa));  // padding too: the argument bytes key the graph cache
    sa.B = p->B; sa.T = p->T; sa.H = p->H; sa.NC = n_chunks(p->T);
    sa.cu = cu;
    sa.c_begin = c0; sa.c_end = c1;
    sa.rec = sb.rec; sa.gC = sb.gC;
    sa.S_in = S_in; sa.S_out = S_out; sa.S_T = S_T; sa.sc = sb.sc;
    return sa;
}

template <class T, int D>
gdn::OutArgs out_args(const gdn_fwd_params *p, int reverse, const ScanBufs &sb, int c0, int mode, float *acc,
                      const int *cu, int t_mid = 0) {
    gdn::OutArgs oa;
    memset(&oa, 0, sizeof(oa));  // padding too: the argument bytes key the graph cache
    oa.B = p->B; oa.T = p->T; oa.H = p->H; oa.NC = n_chunks(p->T); oa.reverse = reverse;
    oa.cu = cu;
    oa.c_begin = c0; oa.mode = mode; oa.t_mid = t_mid;
    oa.rec = sb.rec; oa.sc = sb.sc;
    oa.gate = p->gate; oa.norm_w = p->norm_w; oa.eps = p->eps_norm;
    oa.out = p->o; oa.acc = acc;
    return oa;
}

// Launches woven into a scan's plan (see fwd_call_staged), or none.
struct Staged {
    const std::vector<std::vector<gdn_internal::ExtLaunch>> *post = nullptr;
    int stream = 3;
};

// One scan's range-pipelined launches: preps on `prep_stream`, the state
// chain on `state_stream` (range i waits for prep i), and the output of each
// range on `out_stream` (waits for state i).  out_mode: see OutArgs.  cu: the
// device copy of the sequence table of a variable-length batch, or null.
// staged: launches on staged.stream, post[i] after output i (waiting for it).
template <class T, int D>
void plan_scan(Plan &plan, const gdn_fwd_params *p, int reverse, const ScanBufs &sb, float *S_T, int prep_stream,
               int state_stream, int out_stream, int out_mode, float *acc, const int *cu,
               const Staged &staged = Staged()) {
    const int NC = n_chunks(p->T), R = n_ranges(NC);
    const void *prep = reinterpret_cast<const void *>(&gdn::gdn_prep_kernel<T, D>);
    const void *state = reinterpret_cast<const void *>(&gdn::gdn_state_kernel<T, D>);
    const void *out = reinterpret_cast<const void *>(&gdn::gdn_out_kernel<T, D>);
    std::vector<int> prep_done(R), state_done(R);
    for (int i = 0; i < R; ++i) {
        const int c0 = range_begin(NC, R, i), c1 = range_begin(NC, R, i + 1);
        plan.launch(prep_stream, "gdn_prep_kernel", prep, dim3(c1 - c0, p->H, p->B), dim3(gdn::kThreads),
                    sizeof(gdn::PrepSmem<T, D>), prep_args<T, D>(p, reverse, sb, c0, cu));
        prep_done[i] = plan.record(prep_stream);
    }
    const int used = p->B * p->H * (D / 16);
    for (int i = 0; i < R; ++i) {
        const int c0 = range_begin(NC, R, i), c1 = range_begin(NC, R, i + 1);
        // a sequence that ends in range i writes S_T; the others hand over through smid
        const float *S_in = i == 0 ? p->S0 : sb.smid[(i - 1) & 1];
        float *S_out = i == R - 1 ? nullptr : sb.smid[i & 1];
        plan.wait(state_stream, prep_done[i]);
        plan.launch(state_stream, "gdn_state_kernel", state, dim3((used + 7) / 8 * 8), dim3(gdn::StateCfg<T, D>::THREADS),
                    state_lds<T, D>(), state_args<T, D>(p, sb, c0, c1, S_in, S_out, S_T, cu));
        state_done[i] = plan.record(state_stream);
    }
    for (int i = 0; i < R; ++i) {
        const int c0 = range_begin(NC, R, i), c1 = range_begin(NC, R, i + 1);
        plan.wait(out_stream, state_done[i]);
        plan.launch(out_stream, "gdn_out_kernel", out, dim3(c1 - c0, p->H, p->B), dim3(gdn::kThreads),
                    sizeof(gdn::OutSmem<T, D>), out_args<T, D>(p, reverse, sb, c0, out_mode, acc, cu));
        if (staged.post) {
            plan.wait(staged.stream, plan.record(out_stream));
            for (const gdn_internal::ExtLaunch &e : (*staged.post)[i]) plan.launch_ext(staged.stream, e);
        }
    }
}

// The bidirectional variant: both scans co-scheduled.  The preps of the two
// directions alternate on one stream (forward range 0, reversed range 0,
// forward range 1, ...), so both chains start at once and advance together
// on streams of their own.  The outputs are summed in fp32 and stored once:
// with t_mid the forward scan's chunk boundary nearest the middle, each scan
// is the first to reach one half of the tokens (forward: t < t_mid,
// reversed: t >= t_mid) and writes its normalised output there to the fp32
// accumulator; on the other half it adds the accumulator and stores y.  The
// output launches run on one stream in an order that puts every writer of a
// token after the first writer of that token:
//   1. forward ranges before the middle, interleaved with the reversed ranges
//      whose tokens all lie at or after t_mid;
//   2. the reversed range (if any) that straddles t_mid;
//   3. forward ranges from the middle on, interleaved with the remaining
//      reversed ranges.
// Each also waits for its own chain range.
template <class T, int D>
void plan_bidir(Plan &plan, const gdn_fwd_params *p, float *S_T_rev, const Layout &L) {
    const int NC = n_chunks(p->T), R = n_ranges(NC, kRangeTargetBidir), Tn = p->T;
    const ScanBufs sb[2] = {scan_bufs(p, L, 0), scan_bufs(p, L, 1)};
    float *S_T[2] = {p->S_T, S_T_rev};
    float *acc = gdn_internal::at_offset<float>(p->workspace, L.acc);
    const int chain_stream[2] = {0, 3}, prep_stream = 1, out_stream = 2;
    const int i_mid = R / 2;
    const int t_mid = std::min(Tn, range_begin(NC, R, i_mid) * gdn::kChunk);
    const void *prep = reinterpret_cast<const void *>(&gdn::gdn_prep_kernel<T, D>);
    const void *state = reinterpret_cast<const void *>(&gdn::gdn_state_kernel<T, D>);
    const void *out = reinterpret_cast<const void *>(&gdn::gdn_out_kernel<T, D>);
    std::vector<int> prep_done[2], state_done[2];
    for (int d = 0; d < 2; ++d) {
        prep_done[d].resize(R);
        state_done[d].resize(R);
    }
    for (int i = 0; i < R; ++i) {
        const int c0 = range_begin(NC, R, i), c1 = range_begin(NC, R, i + 1);
        for (int d = 0; d < 2; ++d) {
            plan.launch(prep_stream, "gdn_prep_kernel", prep, dim3(c1 - c0, p->H, p->B), dim3(gdn::kThreads),
                        sizeof(gdn::PrepSmem<T, D>), prep_args<T, D>(p, d, sb[d], c0, nullptr));
            prep_done[d][i] = plan.record(prep_stream);
        }
    }
    const int used = p->B * p->H * (D / 16);
    for (int d = 0; d < 2; ++d) {
        for (int i = 0; i < R; ++i) {
            const int c0 = range_begin(NC, R, i), c1 = range_begin(NC, R, i + 1);
            const float *S_in = i == 0 ? p->S0 : sb[d].smid[(i - 1) & 1];
            float *S_out = i == R - 1 ? nullptr : sb[d].smid[i & 1];
            plan.wait(chain_stream[d], prep_done[d][i]);
            plan.launch(chain_stream[d], "gdn_state_kernel", state, dim3((used + 7) / 8 * 8),
                        dim3(gdn::StateCfg<T, D>::THREADS), state_lds<T, D>(),
                        state_args<T, D>(p, sb[d], c0, c1, S_in, S_out, S_T[d], nullptr));
            state_done[d][i] = plan.record(chain_stream[d]);
        }
    }
    auto out_launch = [&](int d, int i) {
        const int c0 = range_begin(NC, R, i), c1 = range_begin(NC, R, i + 1);
        plan.wait(out_stream, state_done[d][i]);
        plan.launch(out_stream, "gdn_out_kernel", out, dim3(c1 - c0, p->H, p->B), dim3(gdn::kThreads),
                    sizeof(gdn::OutSmem<T, D>), out_args<T, D>(p, d, sb[d], c0, 1, acc, nullptr, t_mid));
    };
    // reversed range j covers sequence positions [T - 64 c1, T - 64 c0)
    std::vector<int> rev_first, rev_mixed, rev_second;
    for (int j = 0; j < R; ++j) {
        const long long lo = (long long)Tn - (long long)gdn::kChunk * range_begin(NC, R, j + 1);
        const long long hi = (long long)Tn - (long long)gdn::kChunk * range_begin(NC, R, j);
        if (lo >= t_mid) rev_first.push_back(j);
        else if (hi <= t_mid) rev_second.push_back(j);
        else rev_mixed.push_back(j);
    }
    for (size_t k = 0; k < (size_t)std::max(i_mid, (int)rev_first.size()); ++k) {
        if ((int)k < i_mid) out_launch(0, (int)k);
        if (k < rev_first.size()) out_launch(1, rev_first[k]);
    }
    for (int j : rev_mixed) out_launch(1, j);
    for (size_t k = 0; k < (size_t)std::max(R - i_mid, (int)rev_second.size()); ++k) {
        if (i_mid + (int)k < R) out_launch(0, i_mid + (int)k);
        if (k < rev_second.size()) out_launch(1, rev_second[k]);
    }
}

template <class T, int D>
gdn_status plan_fwd(Plan &plan, const gdn_fwd_params *p, float *S_T_rev, bool bidir, const int *cu,
                    const Staged &staged) {
    const Layout L = layout(p, bidir ? 2 : 1, cu != nullptr);
    const int start = plan.record(0);
    for (int s = 1; s < kStreams; ++s) plan.wait(s, start);
    if (!bidir) {
        plan_scan<T, D>(plan, p, p->reverse, scan_bufs(p, L, 0), p->S_T, 1, 0, 2, 0, nullptr, cu, staged);
    } else {
        plan_bidir<T, D>(plan, p, S_T_rev, L);
    }
    for (int s = 1; s < kStreams; ++s) plan.wait(0, plan.record(s));
    return GDN_OK;
}

gdn_status make_plan(Plan &plan, const gdn_fwd_params *p, float *S_T_rev, bool bidir, const int *cu = nullptr,
                     const Staged &staged = Staged()) {
    if (p->io_dtype == GDN_BF16 && p->Dk == 128) return plan_fwd<bf16, 128>(plan, p, S_T_rev, bidir, cu, staged);
    if (p->io_dtype == GDN_BF16 && p->Dk == 64) return plan_fwd<bf16, 64>(plan, p, S_T_rev, bidir, cu, staged);
    if (p->io_dtype == GDN_F32 && p->Dk == 128) return plan_fwd<float, 128>(plan, p, S_T_rev, bidir, cu, staged);
    if (p->io_dtype == GDN_F32 && p->Dk == 64) return plan_fwd<float, 64>(plan, p, S_T_rev, bidir, cu, staged);
    return GDN_ERR_UNSUPPORTED;
}

// Kernel attributes (dynamic LDS above 64 KB), set once per process.
gdn_status set_attributes() {
    static std::once_flag once;
    static gdn_status result = GDN_OK;
    std::call_once(once, [] {
        struct A {
            const void *fn;
            size_t lds;
        } attrs[] = {
            {reinterpret_cast<const void *>(&gdn::gdn_prep_kernel<bf16, 128>), sizeof(gdn::PrepSmem<bf16, 128>)},
            {reinterpret_cast<const void *>(&gdn::gdn_prep_kernel<bf16, 64>), sizeof(gdn::PrepSmem<bf16, 64>)},
            {reinterpret_cast<const void *>(&gdn::gdn_prep_kernel<float, 128>), sizeof(gdn::PrepSmem<float, 128>)},
            {reinterpret_cast<const void *>(&gdn::gdn_prep_kernel<float, 64>), sizeof(gdn::PrepSmem<float, 64>)},
            {reinterpret_cast<const void *>(&gdn::gdn_state_kernel<bf16, 128>), state_lds<bf16, 128>()},
            {reinterpret_cast<const void *>(&gdn::gdn_state_kernel<bf16, 64>), state_lds<bf16, 64>()},
            {reinterpret_cast<const void *>(&gdn::gdn_state_kernel<float, 128>), state_lds<float, 128>()},
            {reinterpret_cast<const void *>(&gdn::gdn_state_kernel<float, 64>), state_lds<float, 64>()},
            {reinterpret_cast<const void *>(&gdn::gdn_out_kernel<bf16, 128>), sizeof(gdn::OutSmem<bf16, 128>)},
            {reinterpret_cast<const void *>(&gdn::gdn_out_kernel<bf16, 64>), sizeof(gdn::OutSmem<bf16, 64>)},
            {reinterpret_cast<const void *>(&gdn::gdn_out_kernel<float, 128>), sizeof(gdn::OutSmem<float, 128>)},
            {reinterpret_cast<const void *>(&gdn::gdn_out_kernel<float, 64>), sizeof(gdn::OutSmem<float, 64>)},
        };
        for (const A &a : attrs)
            if (hipFuncSetAttribute(a.fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)a.lds) != hipSuccess)
                result = GDN_ERR_HIP;
    });
    return result;
}

gdn_status call(const gdn_fwd_params *p, float *S_T_rev, bool bidir, hipEvent_t *timing, int n_timing,
                hipStream_t s) {
    if (!sizes_ok(p)) return GDN_ERR_INVALID_ARG;
    gdn_status st = validate(p, S_T_rev, bidir ? 2 : 1, (size_t)p->B * p->T, false);
    if (st != GDN_OK) return st;
    if (bidir && p->reverse != 0) return GDN_ERR_INVALID_ARG;
    Plan plan;
    st = make_plan(plan, p, S_T_rev, bidir);
    if (st != GDN_OK) return st;
    if (timing && n_timing < 2 * (int)plan.launches.size()) return GDN_ERR_INVALID_ARG;
    st = set_attributes();
    if (st != GDN_OK) return st;
    return run_plan(plan, s, timing, !bidir);
}

// Variable-length batch: p->B sequences packed along the token axis,
// sequence b at rows cu[b] .. cu[b+1] - 1 (host table).  Returns the longest
// length in *T_max, or an error for a malformed table.
gdn_status check_seq_table(const gdn_fwd_params *p, const int *cu, int *T_max) {
    if (!p || !cu || p->B < 1) return GDN_ERR_INVALID_ARG;
    if (cu[0] != 0) return GDN_ERR_INVALID_ARG;
    int longest = 0;
    for (int b = 0; b < p->B; ++b) {
        const long long len = (long long)cu[b + 1] - cu[b];
        if (len < 1) return GDN_ERR_INVALID_ARG;  // lengths >= 1, offsets increasing
        if (len > longest) longest = (int)len;
    }
    *T_max = longest;
    return GDN_OK;
}

// The params of a variable-length call with T set to the longest length.
gdn_status varlen_params(const gdn_fwd_params *p, const int *cu, gdn_fwd_params &q) {
    int T_max = 0;
    gdn_status st = check_seq_table(p, cu, &T_max);
    if (st != GDN_OK) return st;
    q = *p;
    q.T = T_max;
    return sizes_ok(&q) ? GDN_OK : GDN_ERR_INVALID_ARG;
}

gdn_status varlen_call(const gdn_fwd_params *p, const int *cu, hipStream_t s) {
    gdn_fwd_params q;
    gdn_status st = varlen_params(p, cu, q);
    if (st != GDN_OK) return st;
    st = validate(&q, nullptr, 1, (size_t)cu[q.B], true);
    if (st != GDN_OK) return st;
    const Layout L = layout(&q, 1, true);
    int *cu_dev = gdn_internal::at_offset<int>(q.workspace, L.seq);
    Plan plan;
    st = make_plan(plan, &q, nullptr, false, cu_dev);
    if (st != GDN_OK) return st;
    st = set_attributes();
    if (st != GDN_OK) return st;
    // the table goes to the workspace first, on the caller's stream
    if (hipMemcpyAsync(cu_dev, cu, sizeof(int) * (q.B + 1), hipMemcpyHostToDevice, s) != hipSuccess)
        return GDN_ERR_HIP;
    return run_plan(plan, s, nullptr, true);
}

// ---- the entry point that allocates nothing (gdn_fwd_noalloc)
//
// Its workspace is this file-scope device array: every GPU the library runs
// on holds its own copy, for the life of the process.  In host code the
// array's name only stands for it; the address of a device's copy is taken
// once per device with hipGetSymbolAddress (with that device current) and
// kept below, and only that address reaches the kernels.  The workspace
// needs no clearing: every byte a call reads was written earlier in the same
// call.  Calls that overlap on one GPU share the array and race.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
std::map<int, void *> g_scratch;  // device -> address of its copy of `scratch`

gdn_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GDN_ERR_HIP;
        it = g_scratch.emplace(dev, ptr).first;
    }
    *out = it->second;
    return GDN_OK;
}

// gdn_fwd's launches in plan order, all on the caller's stream (no library
// streams, events or graphs: nothing is created), with `scratch` as the
// workspace.
gdn_status noalloc_call(const gdn_fwd_params *p, hipStream_t s) {
    if (!sizes_ok(p)) return GDN_ERR_INVALID_ARG;
    gdn_fwd_params q = *p;
    const size_t need = layout(&q, 1).total;
    if (need > kScratchBytes) return GDN_ERR_WORKSPACE;  // beyond the array: refused before any device call
    void *ws = nullptr;
    gdn_status st = scratch_address(&ws);
    if (st != GDN_OK) return st;
    q.workspace = ws;
    q.workspace_bytes = kScratchBytes;
    st = validate(&q, nullptr, 1, (size_t)q.B * q.T, false);
    if (st != GDN_OK) return st;
    Plan plan;
    st = make_plan(plan, &q, nullptr, false);
    if (st != GDN_OK) return st;
    st = set_attributes();
    if (st != GDN_OK) return st;
    // every launch waits for the ones before it on the one stream, which
    // covers each cross-stream dependency of the plan (all preps come before
    // every state launch, and those before every output launch)
    for (const Op &op : plan.ops) {
        if (op.kind != Op::LAUNCH) continue;
        const Launch &L = plan.launches[op.event];
        void *kargs[] = {const_cast<unsigned char *>(L.args)};
        if (hipLaunchKernel(L.fn, L.grid, L.block, kargs, L.smem, s) != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

}  // namespace

gdn_status gdn_internal::fwd_check(const gdn_fwd_params *p) {
    if (!sizes_ok(p)) return GDN_ERR_INVALID_ARG;
    return validate(p, nullptr, 1, (size_t)p->B * p->T, false);
}

gdn_status gdn_internal::fwd_call(const gdn_fwd_params *p, hipEvent_t *timing, int n_timing, hipStream_t s) {
    return call(p, nullptr, false, timing, n_timing, s);
}

void gdn_internal::scan_range_bounds(const gdn_fwd_params *p, std::vector<int> &bounds) {
    const int NC = n_chunks(p->T), R = n_ranges(NC);
    bounds.resize(R + 1);
    for (int i = 0; i <= R; ++i) bounds[i] = range_begin(NC, R, i);
}

gdn_status gdn_internal::fwd_call_staged(const gdn_fwd_params *p, const std::vector<std::vector<ExtLaunch>> &post,
                                         hipStream_t s) {
    if (!sizes_ok(p)) return GDN_ERR_INVALID_ARG;
    gdn_status st = validate(p, nullptr, 1, (size_t)p->B * p->T, false);
    if (st != GDN_OK) return st;
    if ((int)post.size() != n_ranges(n_chunks(p->T))) return GDN_ERR_INVALID_ARG;
    Staged staged;
    staged.post = &post;
    Plan plan;
    st = make_plan(plan, p, nullptr, false, nullptr, staged);
    if (st != GDN_OK) return st;
    st = set_attributes();
    if (st != GDN_OK) return st;
    return run_plan(plan, s, nullptr, true);
}

extern "C" {

size_t gdn_fwd_workspace_bytes(const gdn_fwd_params *p) {
    if (!sizes_ok(p)) return 0;
    return layout(p, 1).total;
}

size_t gdn_fwd_bidir_workspace_bytes(const gdn_fwd_params *p) {
    if (!sizes_ok(p)) return 0;
    return layout(p, 2).total;
}

gdn_status gdn_fwd_noalloc(const gdn_fwd_params *p, struct ihipStream_t *stream) {
    try {
        return noalloc_call(p, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
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

size_t gdn_fwd_varlen_workspace_bytes(const gdn_fwd_params *p, const int *cu_seqlens) {
    try {
        gdn_fwd_params q;
        if (varlen_params(p, cu_seqlens, q) != GDN_OK) return 0;
        return layout(&q, 1, true).total;
    } catch (...) {
        return 0;
    }
}

gdn_status gdn_fwd_varlen(const gdn_fwd_params *p, const int *cu_seqlens, struct ihipStream_t *stream) {
    try {
        return varlen_call(p, cu_seqlens, stream);
    } catch (...) {
        return GDN_ERR_HIP;
    }
}

int gdn_fwd_launch_count(const gdn_fwd_params *p, int bidirectional) {
    if (!sizes_ok(p) || !supported(p)) return -1;
    try {
        Plan plan;
        if (make_plan(plan, p, nullptr, bidirectional != 0) != GDN_OK) return -1;
        return (int)plan.launches.size();
    } catch (...) {
        return -1;
    }
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
    if (!sizes_ok(p) || !supported(p)) return nullptr;
    try {
        Plan plan;
        if (make_plan(plan, p, nullptr, bidirectional != 0) != GDN_OK) return nullptr;
        if (i < 0 || i >= (int)plan.launches.size()) return nullptr;
        return plan.launches[i].name;  // points at a string literal
    } catch (...) {
        return nullptr;
    }
}

const char *gdn_status_string(gdn_status s) {
    // A C caller may pass any int here.  In C++ an enum object holding a
    // value outside the enumeration's range is undefined behaviour, so the
    // code is read as the int it is (host UBSan flags the switch otherwise).
    static_assert(sizeof(gdn_status) == sizeof(int), "gdn_status is passed as an int");
    int code;
    memcpy(&code, &s, sizeof code);
    switch (code) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case GDN_ERR_ALIGNMENT: return "misaligned pointer";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP runtime or launch failure";
    }
    return "unknown status";
}

gdn_status gdn_set_graph_cache_limit(int max_graphs) {
    if (max_graphs < 0 || max_graphs > kMaxCachedGraphs) return GDN_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_graph_limit = (size_t)max_graphs;
    evict_graphs(g_graph_limit);
    if (max_graphs == 0) g_seen.clear();
    return GDN_OK;
}

int gdn_graph_cache_count(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    return (int)g_graphs.size();
}

}  // extern "C"

// kernels.hpp -- HIP kernels (gfx950) of the GDN layer forward.
//
// The layer (LinMorph project page, "Why learn the initialization?": short
// convolutions, update gates, decay terms, normalisation parameters; the
// gated delta rule of the GDN paper, ref. [57] of the VMonarch page, section
// 2) runs as three kernels per scan:
//
//   prep  : one workgroup per (chunk of 64 tokens, head, batch row), all in
//           parallel.  Short conv + SiLU, L2 normalisation, cumulative log
//           decay g, the decayed strictly-lower matrix A (b * K K^T), the
//           solve (I + A) [W | U~] = [diag(b e^g) K | diag(b) V], and the
//           state-independent products Q' = diag(e^g) Q - P W and O0 = P U~
//           with P = (Q K^T o decay), all written to a per-chunk record in
//           MFMA fragment order.
//   state : one workgroup per (16 value channels, head, batch row), walking
//           the chunks in order with its slice of the fp32 state in
//           registers:  U = U~ - W S^T,  S^T <- e^{g_C} S^T + (D K)^T U,
//           D = diag(e^{g_C - g}); it exports each chunk's entry state.
//   out   : one workgroup per (chunk, head, batch row), all in parallel:
//           O = O0 + Q' S^T with the chunk's entry state, then the gated RMS
//           normalisation over all value channels.
//
// The chunked form reproduces the token-by-token recurrence exactly up to
// rounding: inside a chunk, with S0 the entry state, the step is
// S_r = a_r S_{r-1} + u_r k_r^T with u_r = b_r (v_r - a_r S_{r-1} k_r);
// unrolling and substituting gives (I + A) U = diag(b) V - diag(b e^g) K S0^T,
// hence U = U~ - W S0^T, o_r = e^{g_r} S0 q_r + sum_{j<=r} P_rj u_j, and the
// exit state e^{g_C} S0 + U^T D K.  A partial last chunk is padded with
// q = k = v = 0, b = 0, log a = 0, which leaves the state unchanged.
#pragma once
#include <type_traits>

#include "frag.hpp"
#include "sync.hpp"

namespace gdn {

// ------------------------------------------------------------------ layout
// Per-(batch, head, chunk) record, in elements of the operand type T:
//   WN  [w 4][kb D/(4 KPL)][lane 64][KPL]      -W, A operand (rows = tokens 16w..)
//   QP  [w 4][kb D/(4 KPL)][lane 64][KPL]      Q', A operand
//   DKT [w 4][mt D/64][kb 16/KPL][lane 64][KPL] (D K)^T, A operand (rows = key
//                                               channels w*D/4 + 16 mt ..)
//   UT  [vb D/16][w 4][lane 64][4]             U~ in C-tile order
//   O0  [vb D/16][w 4][lane 64][4]             O0 in C-tile order
template <int D> struct Rec {
    static constexpr int WN = 0;
    static constexpr int QP = 64 * D;
    static constexpr int DKT = 128 * D;
    static constexpr int UT = 192 * D;
    static constexpr int O0 = 256 * D;
    static constexpr int SIZE = 320 * D;
};

// Sequences.  Without a table (cu == null) batch row b is a sequence of T
// tokens starting at token row b T.  With one (variable-length batches) the
// tokens of all sequences are packed, sequence b is rows cu[b] .. cu[b+1] - 1,
// T is the longest length and NC = ceil(T / 64) chunks are reserved per
// sequence in the workspace; chunks past a sequence's end do nothing.
struct SeqSpan {
    long long off;  // first token row
    int len;        // tokens
};
__device__ __forceinline__ SeqSpan seq_span(const int *cu, int b, int T) {
    if (cu) {
        const int o = cu[b];
        return SeqSpan{o, cu[b + 1] - o};
    }
    return SeqSpan{(long long)b * T, T};
}

struct PrepArgs {
    int B, T, H, NC, reverse;
    const int *cu;  // sequence table [B + 1] or null
    int c_begin;  // first chunk of this launch (chunk = c_begin + blockIdx.x)
    const void *q, *k, *v;
    const float *log_a, *beta, *conv_q, *conv_k, *conv_v;
    float eps_l2;
    void *rec;   // [B][H][NC] records
    float *gC;   // [B][H][NC] e^{g} at the chunk's last token
};

struct StateArgs {
    int B, T, H, NC;
    const int *cu;       // sequence table [B + 1] or null
    int c_begin, c_end;  // chunks [c_begin, c_end) of the scan
    const void *rec;
    const float *gC;
    const float *S_in;   // [B][H][D][D] state entering chunk c_begin, or null (zeros)
    float *S_out;        // [B][H][D][D] state after chunk c_end - 1 (handed to the next range)
    float *S_T;          // [B][H][D][D] final state of sequences that end in this range, or null
    void *sc;            // [B][H][NC][D/16 value blocks] chunk-entry S^T as B fragments
};

// S^T at the entry of each chunk, as B fragments over the key channels: per
// (batch, head, chunk, value block) KBD fragments of 64 lanes x KPL values.
template <class T, int D> struct ScLayout {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int KBD = D / (4 * KPL);
    static constexpr int PER_VB = KBD * 64 * KPL;  // = 16 * D elements
    static constexpr int PER_CHUNK = (D / 16) * PER_VB;
};

struct OutArgs {
    int B, T, H, NC, reverse;
    const int *cu;      // sequence table [B + 1] or null
    int c_begin;        // chunk = c_begin + blockIdx.x
    int mode;           // 0: write y; 1: bidirectional sum (below)
    // mode 1: the token rows this scan reaches before the other scan does
    // (sequence position t < t_mid for the forward scan, t >= t_mid for the
    // reversed one) write this scan's output to acc (fp32); the others add
    // acc, which the other scan has written, and store y
    int t_mid;
    const void *rec;    // chunk records (QP, O0)
    const void *sc;     // chunk-entry states
    const void *gate;
    const float *norm_w;  // [H][D] or null
    float eps;
    void *out;          // y [B][T][H][D]
    float *acc;         // [B][T][H][D] fp32 (mode 1)
};

// 8 consecutive values as float
__device__ __forceinline__ void load8(const bf16 *p, float *x) {
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    const bf16 *b = reinterpret_cast<const bf16 *>(&u);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)b[i];
}
__device__ __forceinline__ void load8(const float *p, float *x) {
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8(bf16 *p, const float *x) {
    uint4 u;
    bf16 *b = reinterpret_cast<bf16 *>(&u);
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (bf16)x[i];
    *reinterpret_cast<uint4 *>(p) = u;
}
__device__ __forceinline__ void store8(float *p, const float *x) {
    reinterpret_cast<float4 *>(p)[0] = float4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<float4 *>(p)[1] = float4{x[4], x[5], x[6], x[7]};
}
// 4 consecutive values
__device__ __forceinline__ void store4(bf16 *p, floatx4 x) {
    bf16x4 v = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, floatx4 x) { *reinterpret_cast<floatx4 *>(p) = x; }
__device__ __forceinline__ floatx4 load4(const bf16 *p) {
    bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ floatx4 load4(const float *p) { return *reinterpret_cast<const floatx4 *>(p); }
// Streaming (non-temporal) accesses, which do not allocate in L2: for data
// written once and read once much later or by another kernel (the chunk
// records, the output, the bidirectional accumulator) and for data read once
// (the output kernel's records and gate).  This keeps L2 for the state
// chain's operands, which the value-block workgroups of a head share; at
// T = 32760, H = 12, d = 128 the whole call takes 0.670 -> 0.640 ms.
template <class V> __device__ __forceinline__ void st_nt(V *p, const V &v) { __builtin_nontemporal_store(v, p); }
template <class V> __device__ __forceinline__ V ld_nt(const V *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store8_nt(bf16 *p, const float *x) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
    st_nt(reinterpret_cast<bf16x8 *>(p), v);
}
__device__ __forceinline__ void store8_nt(float *p, const float *x) {
    st_nt(reinterpret_cast<floatx4 *>(p), floatx4{x[0], x[1], x[2], x[3]});
    st_nt(reinterpret_cast<floatx4 *>(p) + 1, floatx4{x[4], x[5], x[6], x[7]});
}
__device__ __forceinline__ void store4_nt(bf16 *p, floatx4 x) {
    st_nt(reinterpret_cast<bf16x4 *>(p), bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]});
}
__device__ __forceinline__ void store4_nt(float *p, floatx4 x) { st_nt(reinterpret_cast<floatx4 *>(p), x); }
__device__ __forceinline__ void load8_nt(const bf16 *p, float *x) {
    const bf16x8 v = ld_nt(reinterpret_cast<const bf16x8 *>(p));
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
__device__ __forceinline__ void load8_nt(const float *p, float *x) {
    const floatx4 a = ld_nt(reinterpret_cast<const floatx4 *>(p)), b = ld_nt(reinterpret_cast<const floatx4 *>(p) + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}
__device__ __forceinline__ floatx4 load4_nt(const bf16 *p) {
    const bf16x4 v = ld_nt(reinterpret_cast<const bf16x4 *>(p));
    return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ floatx4 load4_nt(const float *p) { return ld_nt(reinterpret_cast<const floatx4 *>(p)); }
// the same in two steps: the load, and the widening to fp32 when it is used
template <class T> struct Vec4;
template <> struct Vec4<bf16> {
    typedef bf16x4 type;
    static __device__ __forceinline__ floatx4 widen(const type &v) {
        return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
};
template <> struct Vec4<float> {
    typedef floatx4 type;
    static __device__ __forceinline__ floatx4 widen(const type &v) { return v; }
};

// Fragment kb of a row-major row (k contiguous) in tile-chained K order.
__device__ __forceinline__ bf16x8 row_frag(const bf16 *row, int kb, int g) {
    bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + 32 * kb + 4 * g);
    bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + 32 * kb + 16 + 4 * g);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ float row_frag(const float *row, int kb, int g) {
    return row[16 * (kb >> 2) + 4 * g + (kb & 3)];
}

// ====================================================================== prep
// 16 x 16 x 16 products (one 16-token block of the triangular solve).  A K=16
// fragment holds, per lane (r, g), the 4 values k = 4g + e (e = 0..3): one
// bf16 16x16x16 instruction, or four fp32 16x16x4 instructions.
template <class T> struct K16;
template <> struct K16<bf16> {
    typedef bf16x4 frag;
    static __device__ __forceinline__ floatx4 mma(const frag &a, const frag &b, const floatx4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag from4(const floatx4 &x) {
        return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    }
};
template <> struct K16<float> {
    typedef floatx4 frag;
    static __device__ __forceinline__ floatx4 mma(const frag &a, const frag &b, floatx4 c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ frag from4(const floatx4 &x) { return x; }
};

// 8 raw input values of one token row, kept packed until used
template <class T> struct Raw8;
template <> struct Raw8<bf16> {
    uint4 u;
    __device__ __forceinline__ void load(const bf16 *p) { u = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t w = (&u.x)[i >> 1];
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
    }
    __device__ __forceinline__ float get(int i) const { return i < 4 ? (&a.x)[i] : (&b.x)[i - 4]; }
};

template <class T, int D> struct PrepSmem {
    static constexpr int LDX = D + (sizeof(T) == 2 ? 8 : 4);   // q^, k^, v^ rows (later W, Q' staging)
    static constexpr int LDA = 64 + 4;                          // fp32 A rows
    static constexpr int LDP = 64 + (sizeof(T) == 2 ? 8 : 4);   // P rows (P reuses the A storage)
    static constexpr int LDTD = 16 + 4;                         // diagonal inverse rows
    T Qs[64 * LDX];
    T Ks[64 * LDX];
    T Vs[64 * LDX];
    float Am[64 * LDA];
    float Td[4 * 16 * LDTD];
    float g[64], b[64], dk[64], eg[64];
    __device__ T *P() { return reinterpret_cast<T *>(Am); }
};

// Short conv + SiLU (+ L2 normalisation for q and k) of one thread's RUN
// tokens x 8 channels from its raw rows; MASK: positions outside [0, len) are
// zero history and tokens past the sequence's end produce zeros.
template <class T, int D, bool MASK>
__device__ __forceinline__ void conv_silu_norm(const PrepArgs &a, const Raw8<T> (&raw)[3][64 / (kThreads / (D / 8)) + 3],
                                               const bool (&rv)[64 / (kThreads / (D / 8)) + 3],
                                               const float4 *wlds, T *const (&dst)[3], int s0, int cg, int run,
                                               int len) {
    constexpr int G = D / 8;
    constexpr int RUN = 64 / (kThreads / G);
    constexpr int ROWS = RUN + 3;
    constexpr int LDX = PrepSmem<T, D>::LDX;
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        float wt[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 wv = wlds[x * D + 8 * cg + i];
            wt[i][0] = wv.x; wt[i][1] = wv.y; wt[i][2] = wv.z; wt[i][3] = wv.w;
        }
        // the rows widened once, positions outside [0, T) as zeros (the conv's zero history)
        float xr[ROWS][8];
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr)
#pragma unroll
            for (int i = 0; i < 8; ++i) xr[rr][i] = (!MASK || rv[rr]) ? raw[x][rr].get(i) : 0.f;
#pragma unroll
        for (int r = 0; r < RUN; ++r) {
            const bool valid = !MASK || s0 + r < len;
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float s = wt[i][0] * xr[r][i];
#pragma unroll
                for (int j = 1; j < 4; ++j) s = fmaf(wt[i][j], xr[r + j][i], s);
                acc[i] = valid ? silu(s) : 0.f;
            }
            if (x < 2) {
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) ss += acc[i] * acc[i];
                ss = group_sum<G>(ss);
                const float inv = valid ? rsqrt_fast(ss + a.eps_l2) : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= inv;
            }
            T *row = dst[x] + (run * RUN + r) * LDX + 8 * cg;
#pragma unroll
            for (int i = 0; i < 8; ++i) row[i] = (T)acc[i];
        }
    }
}

// Short conv + SiLU (+ L2 normalisation for q and k) of the chunk's 64 scan
// positions into LDS.  Thread layout: G = D/8 threads per token row (8
// channels each); each thread owns RUN consecutive tokens and loads its
// RUN + 3 input rows (3 rows of causal history) once.  Every load of the
// prologue is in flight at once, in this order: the gates (`issue`, wave 0),
// the head's conv weights (copied straight into LDS, into the A storage,
// unused until A is formed), then the raw rows of q, then k, then v.  A
// counted wait then covers the gates and the weight copies only (the RAW_LOADS
// row loads issued after them may still be in flight; the compiler's own
// waits would cover everything, since LDS copies and register loads pending
// together make it wait for zero), `mid` runs, and after the barrier the conv
// of q can start while the rows of k and v arrive.
template <class T, int D> struct PrologueShape {
    static constexpr int G = D / 8;
    static constexpr int RUN = 64 / (kThreads / G);
    static constexpr int ROWS = RUN + 3;
    // vector memory instructions per thread for the raw rows (Raw8::load: one
    // 16-byte load for bf16, two for fp32)
    static constexpr int RAW_LOADS = 3 * ROWS * (sizeof(T) == 2 ? 1 : 2);
    static_assert(RAW_LOADS <= 63, "the counted wait below needs the row loads within the vmcnt range");
};
template <class T, int D, class Issue, class Mid>
__device__ __forceinline__ void prologue(const PrepArgs &a, PrepSmem<T, D> &sm, unsigned char *smem, int c, int h,
                                         SeqSpan sq, Issue issue, Mid mid) {
    typedef PrologueShape<T, D> PS;
    constexpr int G = PS::G, RUN = PS::RUN, ROWS = PS::ROWS;
    const int tid = threadIdx.x, cg = tid % G, run = tid / G;
    const int s0 = c * 64 + run * RUN;
    const T *src[3] = {static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v)};
    T *dst[3] = {sm.Qs, sm.Ks, sm.Vs};
    issue();
    __builtin_amdgcn_sched_barrier(0);
    // weights [3][D][4] fp32: 1 KB units of 64 channels, 16 B per lane
    float4 *wlds = reinterpret_cast<float4 *>(sm.Am);
    {
        constexpr int UNITS = 3 * D / 64;
        const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
        const unsigned char *wl = smem + ((const unsigned char *)wlds - (const unsigned char *)&sm);
#pragma unroll
        for (int u = w; u < UNITS; u += kWaves) {
            const int x = u / (D / 64), ch = (u % (D / 64)) * 64 + lane;
            const float *wsrc = x == 0 ? a.conv_q : (x == 1 ? a.conv_k : a.conv_v);
            __builtin_amdgcn_global_load_lds(wsrc + ((size_t)h * D + ch) * 4, const_cast<unsigned char *>(wl) + u * 1024,
                                             16, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    Raw8<T> raw[3][ROWS];
    bool rv[ROWS];
    size_t off[ROWS];
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) {
        const int sp = s0 - 3 + rr;
        rv[rr] = sp >= 0 && sp < sq.len;
        int si = a.reverse ? sq.len - 1 - sp : sp;
        si = si < 0 ? 0 : (si >= sq.len ? sq.len - 1 : si);
        off[rr] = (((size_t)sq.off + si) * a.H + h) * D + 8 * cg;
    }
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr) raw[x][rr].load(src[x] + off[rr]);
    __builtin_amdgcn_sched_barrier(0);
    // the gates and the weight copies (issued before the RAW_LOADS row loads)
    // have landed; the rows may still be in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PS::RAW_LOADS));
    mid();
    lds_barrier();
    // chunks away from both ends of the sequence need no masking
    if (c > 0 && (c + 1) * 64 <= sq.len)
        conv_silu_norm<T, D, false>(a, raw, rv, wlds, dst, s0, cg, run, sq.len);
    else
        conv_silu_norm<T, D, true>(a, raw, rv, wlds, dst, s0, cg, run, sq.len);
}

template <class T, int D>
__global__ __launch_bounds__(kThreads, 2) void gdn_prep_kernel(PrepArgs a) {
    typedef Mfma<T> M;
    typedef typename M::frag frag;
    typedef K16<T> K;
    typedef typename K::frag kfrag;
    constexpr int KPL = M::KPL;
    constexpr int KBD = D / (4 * KPL);  // fragments over K = D
    constexpr int KBC = 16 / KPL;       // fragments over K = 64
    constexpr int MT = D / 64;
    constexpr int NCT = D / 32;         // 16-column tiles of [W | U~] per wave
    typedef PrepSmem<T, D> SM;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM &sm = *reinterpret_cast<SM *>(smem_raw);

    const int c = a.c_begin + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const SeqSpan sq = seq_span(a.cu, b, a.T);
    if (c * 64 >= sq.len) return;  // past this sequence's end (variable lengths)
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, n = lane % 16, g = lane / 16;

    // ---- gates (b and the cumulative log decay g inside the chunk): loaded
    // first, scanned once the prologue's other loads are issued
    float la = 0.f, be = 0.f;
    auto gates_issue = [&] {
        if (tid < 64) {
            const int s = c * 64 + tid;
            const bool valid = s < sq.len;
            const int src = a.reverse ? sq.len - 1 - s : s;
            la = valid ? a.log_a[((size_t)sq.off + src) * a.H + h] : 0.f;
            be = valid ? a.beta[((size_t)sq.off + src) * a.H + h] : 0.f;
        }
    };
    auto gates = [&] {
        if (tid < 64) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                float y = __shfl_up(la, off, 64);
                if (tid >= off) la += y;
            }
            sm.g[tid] = la;
            sm.b[tid] = be;
            sm.eg[tid] = expf(la);
            sm.dk[tid] = expf(__shfl(la, 63, 64) - la);
        }
    };
    prologue<T, D>(a, sm, smem_raw, c, h, sq, gates_issue, gates);
    __syncthreads();

    // ---- A = strictly lower (b_i e^{g_i - g_j} k_i . k_j), rows 16w.. of this wave
    {
        floatx4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = zero4();
        const T *arow = sm.Ks + (16 * w + n) * SM::LDX;
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            frag fa = row_frag(arow, kb, g);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (t <= w) acc[t] = M::mma(fa, row_frag(sm.Ks + (16 * t + n) * SM::LDX, kb, g), acc[t]);
        }
        // gates into registers first (the stores below may alias them for the compiler)
        float gi[4], bi[4], gj[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            gi[ii] = sm.g[16 * w + 4 * g + ii];
            bi[ii] = sm.b[16 * w + 4 * g + ii];
            gj[ii] = sm.g[16 * ii + n];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * w + 4 * g + ii, j = 16 * t + n;
                sm.Am[i * SM::LDA + j] = (j < i) ? bi[ii] * __expf(gi[ii] - gj[t]) * acc[t][ii] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- inverse of the unit lower diagonal block (I + A_ww), column n on lanes 0..15
    if (g == 0) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == n) ? 1.f : 0.f;
        const float *ab = sm.Am + (16 * w) * SM::LDA + 16 * w;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float acc = x[r];
#pragma unroll
            for (int j = 0; j < r; ++j) acc -= ab[r * SM::LDA + j] * x[j];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Td[(w * 16 + r) * SM::LDTD + n] = x[r];
    }
    __syncthreads();

    // ---- blocked solve (I + A) X = R, R = [diag(b e^g) K | diag(b) V], on this
    // wave's NCT column tiles; block row I: X_I = Tinv_I (R_I - sum_{J<I} A_IJ X_J)
    floatx4 X[4][NCT];
    kfrag Xf[4][NCT];
    // waves 0, 1 own the columns of diag(b e^g) K (W), waves 2, 3 those of diag(b) V (U~)
    const bool wave_k = w < 2;
    // bf16: the identity as a K = 16 B operand (lane (n, g) holds rows 4g..4g+3
    // of column n).  A product with it copies the A operand, read as rows of
    // a row-major tile, into C-tile order; with -I it also negates.  Exact.
    kfrag ident{}, nident{};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ident[e] = (T)(4 * g + e == n ? 1.f : 0.f);
            nident[e] = (T)(4 * g + e == n ? -1.f : 0.f);
        }
    }
    const T *rsrc = wave_k ? sm.Ks : sm.Vs;
    const int col0 = (D / 2) * (w & 1);  // first column of this wave inside K or V
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        kfrag aIJ[4];
#pragma unroll
        for (int J = 0; J < I; ++J) {
            const float *p = sm.Am + (16 * I + n) * SM::LDA + 16 * J + 4 * g;
            floatx4 v = *reinterpret_cast<const floatx4 *>(p);
            aIJ[J] = K::from4(-v);
        }
        const kfrag tI = K::from4(*reinterpret_cast<const floatx4 *>(sm.Td + (16 * I + n) * SM::LDTD + 4 * g));
        float scale[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = 16 * I + 4 * g + ii;
            scale[ii] = wave_k ? sm.b[t] * sm.eg[t] : sm.b[t];
        }
        floatx4 acc[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if constexpr (sizeof(T) == 2) {
                // rows 16I.. of R's columns col0 + 16ct.. into C-tile order
                const kfrag rf = *reinterpret_cast<const kfrag *>(rsrc + (16 * I + n) * SM::LDX + col0 + 16 * ct + 4 * g);
                acc[ct] = K::mma(rf, ident, zero4());
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) acc[ct][ii] *= scale[ii];
            } else {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    acc[ct][ii] = scale[ii] * to_f(rsrc[(16 * I + 4 * g + ii) * SM::LDX + col0 + 16 * ct + n]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int J = 0; J < I; ++J) acc[ct] = K::mma(aIJ[J], Xf[J][ct], acc[ct]);
            X[I][ct] = K::mma(tI, K::from4(acc[ct]), zero4());
            Xf[I][ct] = K::from4(X[I][ct]);
        }
    }
    __syncthreads();

    // ---- P = lower-inclusive (e^{g_r - g_j} q_r . k_j), rows 16w.., into the A storage
    {
        floatx4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = zero4();
        const T *arow = sm.Qs + (16 * w + n) * SM::LDX;
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            frag fa = row_frag(arow, kb, g);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (t <= w) acc[t] = M::mma(fa, row_frag(sm.Ks + (16 * t + n) * SM::LDX, kb, g), acc[t]);
        }
        T *P = sm.P();
        float gi[4], gj[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            gi[ii] = sm.g[16 * w + 4 * g + ii];
            gj[ii] = sm.g[16 * ii + n];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * w + 4 * g + ii, j = 16 * t + n;
                P[i * SM::LDP + j] = (T)((j <= i) ? __expf(gi[ii] - gj[t]) * acc[t][ii] : 0.f);
            }
        }
    }
    __syncthreads();

    // ---- P X on this wave's columns: Q' = e^g Q - P W (W columns), O0 = P U~
    T *rec = static_cast<T *>(a.rec) + (((size_t)b * a.H + h) * a.NC + c) * (size_t)Rec<D>::SIZE;
    if constexpr (sizeof(T) == 2) {
        const T *P = sm.P();
        if (wave_k) {
            // Q'^T = e^g Q^T - W^T P^T, computed transposed so that its C tiles
            // (rows = key channels 4g.., column = token n) are the QP record's
            // A fragments (row = token, K = key channels) without a transpose:
            // the A operand -W^T over tokens is this wave's X tiles (negated),
            // the B operand P^T is read as rows of P.
            frag nxf[2][NCT];  // -W^T fragments over the 64 tokens: kb = 0, 1
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        nxf[kb][ct][e] = (T)(-X[2 * kb][ct][e]);
                        nxf[kb][ct][4 + e] = (T)(-X[2 * kb + 1][ct][e]);
                    }
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                frag pf[KBC];
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) pf[kb] = row_frag(P + (16 * R + n) * SM::LDP, kb, g);
                const float egn = sm.eg[16 * R + n];
                floatx4 qt[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    // e^g Q^T: token 16R + n, key channels col0 + 16ct + 4g.. (C-tile order as read)
                    const kfrag qv = *reinterpret_cast<const kfrag *>(sm.Qs + (16 * R + n) * SM::LDX + col0 + 16 * ct + 4 * g);
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) qt[ct][ii] = egn * to_f(qv[ii]);
#pragma unroll
                    for (int kb = 0; kb < KBC; ++kb) qt[ct] = M::mma(nxf[kb][ct], pf[kb], qt[ct]);
                }
#pragma unroll
                for (int kq = 0; kq < NCT / 2; ++kq) {
                    frag f;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        f[ii] = (T)qt[2 * kq][ii];
                        f[4 + ii] = (T)qt[2 * kq + 1][ii];
                    }
                    st_nt(reinterpret_cast<frag *>(rec + Rec<D>::QP + ((R * KBD + col0 / 32 + kq) * 64 + lane) * KPL), f);
                }
            }
            // WN = -W: the transposes of X's tiles through -I are the A
            // fragments (row = token, K = key channels)
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                floatx4 wt[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) wt[ct] = K::mma(Xf[I][ct], nident, zero4());
#pragma unroll
                for (int kq = 0; kq < NCT / 2; ++kq) {
                    frag f;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        f[ii] = (T)wt[2 * kq][ii];
                        f[4 + ii] = (T)wt[2 * kq + 1][ii];
                    }
                    st_nt(reinterpret_cast<frag *>(rec + Rec<D>::WN + ((I * KBD + col0 / 32 + kq) * 64 + lane) * KPL), f);
                }
            }
        } else {
            // O0 = P U~ and U~, in C-tile order
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                frag pf[KBC];
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) pf[kb] = row_frag(P + (16 * R + n) * SM::LDP, kb, g);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    floatx4 acc = zero4();
#pragma unroll
                    for (int kb = 0; kb < KBC; ++kb) {
                        frag xb;
#pragma unroll
                        for (int j = 0; j < KPL; ++j) {
                            const int e = kb * KPL + j;  // token block e/4, row 4g + e%4
                            fset(xb, j, X[e >> 2][ct][e & 3]);
                        }
                        acc = M::mma(pf[kb], xb, acc);
                    }
                    const int vb = (col0 + 16 * ct) / 16;
                    store4_nt(rec + Rec<D>::O0 + ((vb * 4 + R) * 64 + lane) * 4, acc);
                    store4_nt(rec + Rec<D>::UT + ((vb * 4 + R) * 64 + lane) * 4, X[R][ct]);
                }
            }
        }
        // DKT: A fragments of (D K)^T, rows = key channel w*D/4 + 16 mt + n, K =
        // tokens; the tiles K[tokens 16I.., keys] come into C-tile order through I
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int key0 = w * (D / 4) + 16 * mt;
            floatx4 kt[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const kfrag kf = *reinterpret_cast<const kfrag *>(sm.Ks + (16 * I + n) * SM::LDX + key0 + 4 * g);
                kt[I] = K::mma(kf, ident, zero4());
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) kt[I][ii] *= sm.dk[16 * I + 4 * g + ii];
            }
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                frag f;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    f[ii] = (T)kt[2 * kb][ii];
                    f[4 + ii] = (T)kt[2 * kb + 1][ii];
                }
                st_nt(reinterpret_cast<frag *>(rec + Rec<D>::DKT + (((w * MT + mt) * KBC + kb) * 64 + lane) * KPL), f);
            }
        }
    } else {
        {
            const T *P = sm.P();
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                frag pf[KBC];
#pragma unroll
                for (int kb = 0; kb < KBC; ++kb) pf[kb] = row_frag(P + (16 * R + n) * SM::LDP, kb, g);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    floatx4 acc = zero4();
#pragma unroll
                    for (int kb = 0; kb < KBC; ++kb) {
                        frag xb;
#pragma unroll
                        for (int j = 0; j < KPL; ++j) {
                            const int e = kb * KPL + j;  // token block e/4, row 4g + e%4
                            fset(xb, j, X[e >> 2][ct][e & 3]);
                        }
                        acc = M::mma(pf[kb], xb, acc);
                    }
                    if (wave_k) {
                        // Q' rows 16R + 4g + ii, staged in Qs over the q^ values it replaces
                        const int col = col0 + 16 * ct + n;
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii) {
                            const int t = 16 * R + 4 * g + ii;
                            const float qv = sm.eg[t] * to_f(sm.Qs[t * SM::LDX + col]) - acc[ii];
                            sm.Qs[t * SM::LDX + col] = (T)qv;
                        }
                    } else {
                        const int vb = (col0 + 16 * ct) / 16;
                        store4_nt(rec + Rec<D>::O0 + ((vb * 4 + R) * 64 + lane) * 4, acc);
                        store4_nt(rec + Rec<D>::UT + ((vb * 4 + R) * 64 + lane) * 4, X[R][ct]);
                    }
                }
            }
            // -W staged row-major in Vs (v^ is no longer needed)
            if (wave_k) {
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii)
                            sm.Vs[(16 * I + 4 * g + ii) * SM::LDX + col0 + 16 * ct + n] = (T)(-X[I][ct][ii]);
            }
        }
        __syncthreads();

        // ---- QP and WN as A fragments: rows = tokens 16w + n, K = key channels (chained)
        {
            const T *qrow = sm.Qs + (16 * w + n) * SM::LDX;
            const T *wrow = sm.Vs + (16 * w + n) * SM::LDX;
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb) {
                st_nt(reinterpret_cast<frag *>(rec + Rec<D>::QP + ((w * KBD + kb) * 64 + lane) * KPL), row_frag(qrow, kb, g));
                st_nt(reinterpret_cast<frag *>(rec + Rec<D>::WN + ((w * KBD + kb) * 64 + lane) * KPL), row_frag(wrow, kb, g));
            }
        }
        // DKT: A fragments of (D K)^T, rows = key channel w*D/4 + 16 mt + n, K = tokens
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int dkc = w * (D / 4) + 16 * mt + n;
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                frag f;
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    const int tok = kchain(kb * KPL + j, g);
                    fset(f, j, sm.dk[tok] * to_f(sm.Ks[tok * SM::LDX + dkc]));
                }
                st_nt(reinterpret_cast<frag *>(rec + Rec<D>::DKT + (((w * MT + mt) * KBC + kb) * 64 + lane) * KPL), f);
            }
        }
    }
    if (tid == 0) a.gC[((size_t)b * a.H + h) * a.NC + c] = sm.eg[63];
}

// ===================================================================== state
// Shape of the state kernel.  NW compute waves split the key channels
// (KQ = D / NW each); the per-chunk U is reduced across them through LDS.
template <class T, int D> struct StateCfg {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int KBD = D / (4 * KPL);                    // fragments over K = D
    static constexpr int KBC = 16 / KPL;                         // fragments over K = 64 tokens
    static constexpr int NW = (sizeof(T) == 2 && D == 64) ? 2 : 4;
    static constexpr int KQ = D / NW;                            // key channels per wave
    static constexpr int KBQ = KQ / (4 * KPL);                   // fragments over a wave's key channels
    static constexpr int MQ = KQ / 16;                           // 16-row tiles of S^T per wave
    static constexpr int TPW = 4 / NW;                           // token tiles each wave reduces
    static constexpr int NB = 4;                                 // chunks of operands held in registers
    static constexpr int THREADS = 64 * NW;
    static_assert(KBQ >= 1 && KQ % (4 * KPL) == 0 && MQ >= 1, "state kernel shape");
};
constexpr int kStateMaxRange = 512;  // chunks per launch (e^{g_C} of the range is staged in LDS)

template <class T, int D> struct StateSmem {
    typedef StateCfg<T, D> C;
    floatx4 part[C::NW][4][64];  // partial U of every wave, per token tile, fp32
    T ub[64 * 16];                 // U as B fragments over the 64 tokens, per lane
    float gcs[kStateMaxRange];     // e^{g_C} of the range's chunks
};

// Operands of one chunk held by one compute wave: -W over its key channels
// for the 4 token tiles, its rows of (D K)^T, and U~ of the tiles it reduces.
template <class T, int D> struct StateOps {
    typedef StateCfg<T, D> C;
    typedef typename Mfma<T>::frag frag;
    frag wf[4][C::KBQ];
    frag dkf[C::MQ][C::KBC];
    typename Vec4<T>::type ut[C::TPW];
};

// One workgroup owns a block of 16 value channels of one head and walks the
// chunks [c_begin, c_end).  Compute wave w keeps S^T rows w KQ .. (w+1) KQ - 1
// (fp32, in registers) and, per chunk:
//   A: stores its rows of the chunk-entry state for the output kernel, and
//      forms its partial -W[:, rows] S^T[rows] for all 4 token tiles,
//      publishing them in LDS;                                   barrier;
//   B: adds U~ and the partials of its token tiles into U, stored as
//      bf16/fp32 B fragments in LDS;                             barrier;
//   C: S^T[rows] <- e^{g_C} S^T[rows] + (D K)^T[rows] U (the decay applied
//      in phase A).
// Its operand fragments come straight from the chunk records in HBM into
// registers, NB chunks ahead (four register sets used in turn; a set's -W
// and U~ are reloaded right after phase A has used them, before the first
// barrier's wait, its (D K)^T after phase C); LDS holds only the exchange.
// Every wave passes 1 + 2 * chunks barriers.
template <class T, int D>
__global__ __launch_bounds__((StateCfg<T, D>::THREADS)) void gdn_state_kernel(StateArgs a) {
    typedef Mfma<T> M;
    typedef typename M::frag frag;
    typedef StateCfg<T, D> C;
    typedef StateOps<T, D> Ops;
    constexpr int KPL = C::KPL, KBD = C::KBD, KBC = C::KBC, KBQ = C::KBQ, MQ = C::MQ, TPW = C::TPW;
    constexpr int NV = D / 16;
    __shared__ StateSmem<T, D> sm;

    // work list: (batch*head, value block) pairs, head-major, so the value
    // blocks of one head share an XCD's L2 for the head's chunk records
    int p;
    if (!xcd_position(blockIdx.x, a.B * a.H * NV, gridDim.x, p)) return;
    // The chain is the critical path of the whole call and shares its CUs
    // with prep and output workgroups: its waves win the instruction issue
    // arbitration on their SIMDs (measured: 0.795 -> 0.776 ms per call).
    __builtin_amdgcn_s_setprio(3);
    const int vb = p % NV;
    const size_t bh = p / NV;
    const int tid = threadIdx.x, lane = tid % 64, n = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);  // (visibly) wave-uniform
    const int vcol = 16 * vb + n;
    const T *rec0 = static_cast<const T *>(a.rec) + bh * a.NC * (size_t)Rec<D>::SIZE;
    const int row0 = w * C::KQ;  // first key channel of this wave
    // this sequence's chunks in the range (variable lengths: possibly none)
    const int nc_seq = (seq_span(a.cu, (int)(bh / a.H), a.T).len + 63) / 64;
    const int c_end = min(a.c_end, nc_seq);
    if (a.c_begin >= c_end) return;

    // e^{g_C} of the range into LDS
    for (int i = tid; i < c_end - a.c_begin; i += C::THREADS) sm.gcs[i] = a.gC[bh * a.NC + a.c_begin + i];

    Ops ops[C::NB];
    auto load_w = [&](Ops &o, int c) {
        const T *rec = rec0 + (size_t)c * Rec<D>::SIZE;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int kb = 0; kb < KBQ; ++kb)
                o.wf[tt][kb] = *reinterpret_cast<const frag *>(rec + Rec<D>::WN + ((tt * KBD + w * KBQ + kb) * 64 + lane) * KPL);
#pragma unroll
        for (int j = 0; j < TPW; ++j)
            o.ut[j] = *reinterpret_cast<const typename Vec4<T>::type *>(rec + Rec<D>::UT + ((vb * 4 + w * TPW + j) * 64 + lane) * 4);
    };
    auto load_dk = [&](Ops &o, int c) {
        const T *rec = rec0 + (size_t)c * Rec<D>::SIZE;
#pragma unroll
        for (int mt = 0; mt < MQ; ++mt)
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb)
                o.dkf[mt][kb] = *reinterpret_cast<const frag *>(rec + Rec<D>::DKT + (((w * MQ + mt) * KBC + kb) * 64 + lane) * KPL);
    };
    auto load_ops = [&](Ops &o, int c) {
        load_w(o, c);
        load_dk(o, c);
    };

    floatx4 S[MQ];
#pragma unroll
    for (int mt = 0; mt < MQ; ++mt)
        S[mt] = a.S_in ? *reinterpret_cast<const floatx4 *>(a.S_in + (bh * D + vcol) * D + row0 + 16 * mt + 4 * g) : zero4();
    T *sc_base = static_cast<T *>(a.sc) + (bh * a.NC * NV + vb) * (size_t)ScLayout<T, D>::PER_VB;

    const int last = c_end - 1;
#pragma unroll
    for (int j = 0; j < C::NB; ++j) load_ops(ops[j], min(a.c_begin + j, last));
    lds_barrier();  // e^{g_C} staged

    auto step = [&](Ops &o, int c) {
        const float gc = sm.gcs[c - a.c_begin];
        // ---- A: entry state out, partial U
        frag sB[KBQ];
#pragma unroll
        for (int kb = 0; kb < KBQ; ++kb)
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const int e = kb * KPL + j;
                fset(sB[kb], j, S[e >> 2][e & 3]);
            }
        // the decay of the update, applied while the entry state is at hand
        // (off the path from the second barrier to the next chunk)
#pragma unroll
        for (int mt = 0; mt < MQ; ++mt) S[mt] *= gc;
        T *scp = sc_base + (size_t)c * NV * ScLayout<T, D>::PER_VB;
#pragma unroll
        for (int kb = 0; kb < KBQ; ++kb)
            *reinterpret_cast<frag *>(scp + ((w * KBQ + kb) * 64 + lane) * KPL) = sB[kb];
        floatx4 up[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            up[tt] = zero4();
#pragma unroll
            for (int kb = 0; kb < KBQ; ++kb) up[tt] = M::mma(o.wf[tt][kb], sB[kb], up[tt]);
            sm.part[w][tt][lane] = up[tt];
        }
        // U~ of this wave's token tiles, widened before its registers are reloaded
        floatx4 uw[TPW];
#pragma unroll
        for (int j = 0; j < TPW; ++j) uw[j] = Vec4<T>::widen(o.ut[j]);
        // this register set's -W and U~ now take chunk c + NB (issued before the barrier wait)
        load_w(o, min(c + C::NB, last));
        lds_barrier();
        // ---- B: U for this wave's token tiles: U~ plus every wave's partial
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tt = w * TPW + j;
            floatx4 u = uw[j];
#pragma unroll
            for (int w2 = 0; w2 < C::NW; ++w2) u += sm.part[w2][tt][lane];
            store4(&sm.ub[lane * 16 + 4 * tt], u);
        }
        lds_barrier();
        // ---- C: S^T[rows] <- e^{g_C} S^T[rows] + (D K)^T[rows] U
        frag uB[KBC];
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb) uB[kb] = *reinterpret_cast<const frag *>(&sm.ub[lane * 16 + kb * KPL]);
#pragma unroll
        for (int mt = 0; mt < MQ; ++mt)
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) S[mt] = M::mma(o.dkf[mt][kb], uB[kb], S[mt]);
        // and its (D K)^T (past the range: the last chunk again, unused)
        load_dk(o, min(c + C::NB, last));
    };
    // whole groups of NB chunks (one back edge, so the loads in flight at the
    // top of the loop are the same on every entry), then the rest
    const int n_ch = c_end - a.c_begin, full = n_ch / C::NB * C::NB;
    for (int c = a.c_begin; c < a.c_begin + full; c += C::NB) {
#pragma unroll
        for (int j = 0; j < C::NB; ++j) step(ops[j], c + j);
    }
#pragma unroll
    for (int j = 0; j < C::NB - 1; ++j)
        if (full + j < n_ch) step(ops[j], a.c_begin + full + j);
    // the sequence's final state if it ends in this range, else the hand-off
    float *S_dst = c_end == nc_seq ? a.S_T : a.S_out;
    if (S_dst) {
#pragma unroll
        for (int mt = 0; mt < MQ; ++mt)
            *reinterpret_cast<floatx4 *>(S_dst + (bh * D + vcol) * D + row0 + 16 * mt + 4 * g) = S[mt];
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ======================================================================= out
template <class T, int D> struct OutSmem {
    static constexpr int LDO = D + 4;  // fp32 rows of O
    T sc[ScLayout<T, D>::PER_CHUNK];  // entry state of every value block, as B fragments
    float Os[64 * LDO];
};

template <class T, int D>
__global__ __launch_bounds__(kThreads, 2) void gdn_out_kernel(OutArgs a) {
    typedef Mfma<T> M;
    typedef typename M::frag frag;
    typedef ScLayout<T, D> SL;
    constexpr int KPL = M::KPL;
    constexpr int KBD = D / (4 * KPL);
    constexpr int NV = D / 16;
    typedef OutSmem<T, D> SM;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM &sm = *reinterpret_cast<SM *>(smem_raw);

    const int c = a.c_begin + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const SeqSpan sq = seq_span(a.cu, b, a.T);
    if (c * 64 >= sq.len) return;  // past this sequence's end (variable lengths)
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, n = lane % 16, g = lane / 16;
    const size_t bh = (size_t)b * a.H + h;

    // stage the chunk-entry state of all value blocks: direct-to-LDS copies
    // of 1 KB units (16 B per lane), all in flight with the loads below
    {
        const unsigned char *src = reinterpret_cast<const unsigned char *>(
            static_cast<const T *>(a.sc) + (bh * a.NC + c) * (size_t)SL::PER_CHUNK);
        constexpr int UNITS = SL::PER_CHUNK * (int)sizeof(T) / 1024;
        static_assert(UNITS % kWaves == 0, "state staging units per wave");
#pragma unroll
        for (int j = 0; j < UNITS / kWaves; ++j) {
            const int u = w + j * kWaves;
            __builtin_amdgcn_global_load_lds(src + u * 1024 + lane * 16, smem_raw + u * 1024, 16, 0, 0);
        }
    }
    const T *rec = static_cast<const T *>(a.rec) + (bh * a.NC + c) * (size_t)Rec<D>::SIZE;
    frag qp[KBD];
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb)
        qp[kb] = ld_nt(reinterpret_cast<const frag *>(rec + Rec<D>::QP + ((w * KBD + kb) * 64 + lane) * KPL));
    floatx4 o[NV];
#pragma unroll
    for (int vb = 0; vb < NV; ++vb) o[vb] = load4_nt(rec + Rec<D>::O0 + ((vb * 4 + w) * 64 + lane) * 4);
    // the gate (and, summing the second scan, the first scan's output) of the
    // rows this thread normalises below, loaded with the rest (rows clamped)
    constexpr int G = D / 8;
    constexpr int TPP = kThreads / G;
    constexpr int PASSES = 64 / TPP;
    const int cg = tid % G;
    size_t roff[PASSES];
    bool first[PASSES];  // mode 1: this scan reaches the row first (writes acc)
    float gv[PASSES][8], prev[PASSES][8];
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        const int s = c * 64 + pass * TPP + tid / G;
        const int sc_ = s < sq.len ? s : sq.len - 1;
        const int t = a.reverse ? sq.len - 1 - sc_ : sc_;
        roff[pass] = (((size_t)sq.off + t) * a.H + h) * D + 8 * cg;
        load8_nt(static_cast<const T *>(a.gate) + roff[pass], gv[pass]);
        first[pass] = a.reverse ? t >= a.t_mid : t < a.t_mid;
        if (a.mode == 1 && !first[pass]) load8_nt(a.acc + roff[pass], prev[pass]);
    }
    float wv[8];  // norm weights (4-byte aligned)
    if (a.norm_w) {
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[i] = a.norm_w[h * D + 8 * cg + i];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[i] = 1.f;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's copies have landed
    __syncthreads();
    // O = O0 + Q' S^T for tokens 16w.., all value channels
#pragma unroll
    for (int vb = 0; vb < NV; ++vb) {
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb)
            o[vb] = M::mma(qp[kb], *reinterpret_cast<const frag *>(sm.sc + ((vb * KBD + kb) * 64 + lane) * KPL),
                           o[vb]);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sm.Os[(16 * w + 4 * g + ii) * SM::LDO + 16 * vb + n] = o[vb][ii];
    }
    __syncthreads();

    // gated RMS normalisation: G threads per token row, 8 channels each
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        const int r = pass * TPP + tid / G;
        const int s = c * 64 + r;
        const bool live = s < sq.len;
        const float *orow = sm.Os + r * SM::LDO + 8 * cg;
        float ov[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ov[i] = orow[i];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += ov[i] * ov[i];
        ss = group_sum<G>(ss);
        const float inv = rsqrt_fast(ss * (1.0f / D) + a.eps);
        if (!live) continue;
        const size_t off = roff[pass];
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = ov[i] * inv * wv[i] * silu(gv[pass][i]);
        if (a.mode == 1 && first[pass]) {
            store8_nt(a.acc + off, y);
        } else {
            if (a.mode == 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] += prev[pass][i];
            }
            store8_nt(static_cast<T *>(a.out) + off, y);
        }
    }
}

}  // namespace gdn

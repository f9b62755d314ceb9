// kernels.hpp -- HIP kernels (gfx950) of the GDN layer forward.
//
// The layer (LinMorph project page, "Why learn the initialization?": short
// convolutions, update gates, decay terms, normalisation parameters; the
// gated delta rule of the GDN paper, ref. [57] of the VMonarch page, section
// 2) runs as three launches per scan:
//
//   prep  : one workgroup per (chunk of 64 tokens, head, batch row), all in
//           parallel.  Short conv + SiLU, L2 normalisation, cumulative log
//           decay g, the decayed strictly-lower matrix A (b * K K^T), the
//           solve (I + A) [W | U~] = [diag(b e^g) K | diag(b) V] by forward
//           substitution, and the state-independent products
//           Q' = diag(e^g) Q - P W and O0 = P U~ with P = (Q K^T o decay),
//           all written to a per-chunk record in MFMA fragment order.
//   state : one workgroup per (16 value channels, head, batch row), walking
//           the chunks in order with its slice of the fp32 state in
//           registers:  U = U~ - W S^T,  O = O0 + Q' S^T,
//                       S^T <- e^{g_C} S^T + (D K)^T U,  D = diag(e^{g_C - g}).
//   norm  : gated RMS normalisation of O over all value channels.
//
// The chunked form reproduces the token-by-token recurrence exactly up to
// rounding: inside a chunk, with S0 the entry state, the step is
// S_r = a_r S_{r-1} + u_r k_r^T with u_r = b_r (v_r - a_r S_{r-1} k_r);
// unrolling and substituting gives (I + A) U = diag(b) V - diag(b e^g) K S0^T,
// hence U = U~ - W S0^T, o_r = e^{g_r} S0 q_r + sum_{j<=r} P_rj u_j, and the
// exit state e^{g_C} S0 + U^T D K.  A partial last chunk is padded with
// q = k = v = 0, b = 0, log a = 0, which leaves the state unchanged.
#pragma once
#include "frag.hpp"

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

struct PrepArgs {
    int B, T, H, NC, reverse;
    const void *q, *k, *v;
    const float *log_a, *beta, *conv_q, *conv_k, *conv_v;
    float eps_l2;
    void *rec;   // [B][H][NC] records
    float *gC;   // [B][H][NC] e^{g} at the chunk's last token
};

struct StateArgs {
    int B, T, H, NC;
    const void *rec;
    const float *gC;
    const float *S0;  // [B][H][D][D] or null
    float *S_T;       // [B][H][D][D] or null
    float *ows;       // [B][H][NC*64][D] unnormalised o, scan order
    float *ps;        // [B][H][D/16][NC*64] partial sums of o^2 per 16 channels
};

struct NormArgs {
    int B, T, H, NC, reverse;
    const float *ows, *ps;      // first (or only) scan
    const float *ows2, *ps2;    // time-reversed scan, or null
    const void *gate;
    const float *norm_w;        // [H][D] or null
    float eps;
    void *out;
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
template <class T, int D> struct PrepSmem {
    static constexpr int LDX = D + (sizeof(T) == 2 ? 8 : 4);   // q^, k^, v^ rows
    static constexpr int LDA = 64 + 4;                          // fp32 A rows
    static constexpr int LDP = 64 + (sizeof(T) == 2 ? 8 : 4);   // P rows
    static constexpr int LDT = 64 + (sizeof(T) == 2 ? 8 : 4);   // [W | U~]^T rows
    T Qs[64 * LDX];
    T Ks[64 * LDX];
    T Vs[64 * LDX];
    float As[64 * LDA];
    T Ps[64 * LDP];
    T XsT[2 * D * LDT];
    float g[64], b[64], dk[64];
};

template <class T, int D>
__device__ __forceinline__ void prologue_tensor(const PrepArgs &a, const T *x, const float *w, T *dst,
                                                bool normalize, int c, int h, int b) {
    constexpr int G = D / 8;           // threads per token (8 channels each)
    constexpr int TPP = kThreads / G;  // tokens per pass
    constexpr int LDX = PrepSmem<T, D>::LDX;
    const int tid = threadIdx.x;
    const int cg = tid % G, tr = tid / G;
    float wt[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float4 wv = reinterpret_cast<const float4 *>(w)[(size_t)h * D + 8 * cg + i];
        wt[i][0] = wv.x; wt[i][1] = wv.y; wt[i][2] = wv.z; wt[i][3] = wv.w;
    }
#pragma unroll
    for (int pass = 0; pass < 64 / TPP; ++pass) {
        const int r = pass * TPP + tr;
        const int s = c * 64 + r;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        const bool valid = s < a.T;
        if (valid) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sp = s - 3 + j;
                if (sp >= 0) {
                    const int src = a.reverse ? a.T - 1 - sp : sp;
                    float xv[8];
                    load8(x + (((size_t)b * a.T + src) * a.H + h) * D + 8 * cg, xv);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] += wt[i][j] * xv[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = silu(acc[i]);
        }
        if (normalize) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += acc[i] * acc[i];
#pragma unroll
            for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
            const float inv = valid ? 1.0f / sqrtf(ss + a.eps_l2) : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] *= inv;
        }
        T *row = dst + r * LDX + 8 * cg;
#pragma unroll
        for (int i = 0; i < 8; ++i) row[i] = (T)acc[i];
    }
}

template <class T, int D>
__global__ __launch_bounds__(kThreads) void gdn_prep_kernel(PrepArgs a) {
    typedef Mfma<T> M;
    typedef typename M::frag frag;
    constexpr int KPL = M::KPL;
    constexpr int KBD = D / (4 * KPL);  // fragments over K = D
    constexpr int KBC = 16 / KPL;       // fragments over K = 64
    constexpr int NT = D / 16;
    constexpr int MT = D / 64;
    typedef PrepSmem<T, D> SM;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SM &sm = *reinterpret_cast<SM *>(smem_raw);

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, n = lane % 16, g = lane / 16;

    // ---- gates: b, cumulative log decay g within the chunk
    if (tid < 64) {
        const int s = c * 64 + tid;
        const bool valid = s < a.T;
        const int src = a.reverse ? a.T - 1 - s : s;
        float la = valid ? a.log_a[((size_t)b * a.T + src) * a.H + h] : 0.f;
        float be = valid ? a.beta[((size_t)b * a.T + src) * a.H + h] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            float y = __shfl_up(la, off, 64);
            if (tid >= off) la += y;
        }
        sm.g[tid] = la;
        sm.b[tid] = be;
    }
    // ---- prologue
    prologue_tensor<T, D>(a, static_cast<const T *>(a.q), a.conv_q, sm.Qs, true, c, h, b);
    prologue_tensor<T, D>(a, static_cast<const T *>(a.k), a.conv_k, sm.Ks, true, c, h, b);
    prologue_tensor<T, D>(a, static_cast<const T *>(a.v), a.conv_v, sm.Vs, false, c, h, b);
    __syncthreads();
    if (tid < 64) sm.dk[tid] = expf(sm.g[63] - sm.g[tid]);

    // ---- K K^T and Q K^T for rows 16w..16w+15 (this wave), all 64 columns
    {
        floatx4 accK[4], accQ[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) { accK[t] = zero4(); accQ[t] = zero4(); }
        const T *arowK = sm.Ks + (16 * w + n) * SM::LDX;
        const T *arowQ = sm.Qs + (16 * w + n) * SM::LDX;
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            frag aK = row_frag(arowK, kb, g);
            frag aQ = row_frag(arowQ, kb, g);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                frag bK = row_frag(sm.Ks + (16 * t + n) * SM::LDX, kb, g);
                accK[t] = M::mma(aK, bK, accK[t]);
                accQ[t] = M::mma(aQ, bK, accQ[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * w + 4 * g + ii, j = 16 * t + n;
                const float gi = sm.g[i], gj = sm.g[j];
                const float dec = (j <= i) ? expf(gi - gj) : 0.f;
                sm.As[i * SM::LDA + j] = (j < i) ? sm.b[i] * dec * accK[t][ii] : 0.f;
                sm.Ps[i * SM::LDP + j] = (T)(dec * accQ[t][ii]);
            }
        }
    }
    __syncthreads();

    // ---- forward substitution: column tid of (I + A) X = [diag(b e^g) K | diag(b) V]
    if (tid < 2 * D) {
        float x[64];
        const bool isK = tid < D;
        const int cc = isK ? tid : tid - D;
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const float rhs = isK ? to_f(sm.Ks[i * SM::LDX + cc]) * expf(sm.g[i])
                                  : to_f(sm.Vs[i * SM::LDX + cc]);
            x[i] = sm.b[i] * rhs;
        }
#pragma unroll
        for (int i = 1; i < 64; ++i) {
            const float *arow = sm.As + i * SM::LDA;
            float acc = x[i];
#pragma unroll
            for (int j = 0; j < i; ++j) acc -= arow[j] * x[j];
            x[i] = acc;
        }
        T *dst = sm.XsT + tid * SM::LDT;
#pragma unroll
        for (int i = 0; i < 64; ++i) dst[i] = (T)x[i];
    }
    __syncthreads();

    // ---- Q' = e^g Q - P W and O0 = P U~ for rows 16w.. (C tiles over D columns)
    floatx4 accW[NT], accU[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) { accW[t] = zero4(); accU[t] = zero4(); }
    {
        const T *prow = sm.Ps + (16 * w + n) * SM::LDP;
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb) {
            frag aP = row_frag(prow, kb, g);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                frag bW = row_frag(sm.XsT + (16 * t + n) * SM::LDT, kb, g);
                frag bU = row_frag(sm.XsT + (D + 16 * t + n) * SM::LDT, kb, g);
                accW[t] = M::mma(aP, bW, accW[t]);
                accU[t] = M::mma(aP, bU, accU[t]);
            }
        }
    }
    T *rec = static_cast<T *>(a.rec) + (((size_t)b * a.H + h) * a.NC + c) * (size_t)Rec<D>::SIZE;
    // O0 and U~ in C-tile order: [vb][w][lane][4], tokens 16w + 4g + ii, channel 16 vb + n
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        store4(rec + Rec<D>::O0 + ((t * 4 + w) * 64 + lane) * 4, accU[t]);
        const T *src = sm.XsT + (D + 16 * t + n) * SM::LDT + 16 * w + 4 * g;
        floatx4 u = floatx4{to_f(src[0]), to_f(src[1]), to_f(src[2]), to_f(src[3])};
        store4(rec + Rec<D>::UT + ((t * 4 + w) * 64 + lane) * 4, u);
    }
    // Q' = e^{g_r} q_r - (P W)_r, written back over this wave's own rows of Qs
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int r = 16 * w + 4 * g + ii, col = 16 * t + n;
            accW[t][ii] = expf(sm.g[r]) * to_f(sm.Qs[r * SM::LDX + col]) - accW[t][ii];
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int r = 16 * w + 4 * g + ii, col = 16 * t + n;
            sm.Qs[r * SM::LDX + col] = (T)accW[t][ii];
        }
    }
    __syncthreads();
    // QP and WN as A fragments: rows 16w + n, K = key channels in chained order
    {
        const T *qrow = sm.Qs + (16 * w + n) * SM::LDX;
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            frag fq = row_frag(qrow, kb, g);
            frag fw;
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const int kk = kchain(kb * KPL + j, g);
                fset(fw, j, -to_f(sm.XsT[kk * SM::LDT + 16 * w + n]));
            }
            *reinterpret_cast<frag *>(rec + Rec<D>::QP + ((w * KBD + kb) * 64 + lane) * KPL) = fq;
            *reinterpret_cast<frag *>(rec + Rec<D>::WN + ((w * KBD + kb) * 64 + lane) * KPL) = fw;
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
            *reinterpret_cast<frag *>(rec + Rec<D>::DKT + (((w * MT + mt) * KBC + kb) * 64 + lane) * KPL) = f;
        }
    }
    if (tid == 0) a.gC[((size_t)b * a.H + h) * a.NC + c] = expf(sm.g[63]);
}

// ===================================================================== state
template <class T, int D> struct StateSmem {
    static constexpr int LDS_S = D / 4 + (sizeof(T) == 2 ? 8 : 4);
    static constexpr int LDS_U = 16 + (sizeof(T) == 2 ? 8 : 4);
    T Sx[64 * LDS_S];  // S^T as B fragments, per lane
    T Ux[64 * LDS_U];  // U as B fragments, per lane
};

template <class T, int D>
__global__ __launch_bounds__(kThreads) void gdn_state_kernel(StateArgs a) {
    typedef Mfma<T> M;
    typedef typename M::frag frag;
    constexpr int KPL = M::KPL;
    constexpr int KBD = D / (4 * KPL);
    constexpr int KBC = 16 / KPL;
    constexpr int MT = D / 64;
    constexpr int NV = D / 16;
    typedef StateSmem<T, D> SM;
    __shared__ SM sm;

    const int vb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, n = lane % 16, g = lane / 16;
    const int vcol = 16 * vb + n;
    const size_t bh = (size_t)b * a.H + h;

    // S^T slice: rows (key channels) w*D/4 + 16 mt + 4g + ii, column vcol
    floatx4 S[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        if (a.S0)
            S[mt] = *reinterpret_cast<const floatx4 *>(a.S0 + (bh * D + vcol) * D + w * (D / 4) + 16 * mt + 4 * g);
        else
            S[mt] = zero4();
    }
    const T *rec0 = static_cast<const T *>(a.rec) + bh * a.NC * (size_t)Rec<D>::SIZE;
    T *sx = sm.Sx + lane * SM::LDS_S;
    T *ux = sm.Ux + lane * SM::LDS_U;

    for (int c = 0; c < a.NC; ++c) {
        const T *rec = rec0 + (size_t)c * Rec<D>::SIZE;
        // publish this wave's part of S^T (elements e = 4 (w MT + mt) + ii)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sx[4 * (w * MT + mt) + ii] = (T)S[mt][ii];
        __syncthreads();
        frag sB[KBD];
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) sB[kb] = *reinterpret_cast<const frag *>(sx + kb * KPL);
        // U = U~ + WN S^T and O = O0 + Q' S^T for tokens 16w..16w+15
        floatx4 u = load4(rec + Rec<D>::UT + ((vb * 4 + w) * 64 + lane) * 4);
        floatx4 o = load4(rec + Rec<D>::O0 + ((vb * 4 + w) * 64 + lane) * 4);
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            frag fw = *reinterpret_cast<const frag *>(rec + Rec<D>::WN + ((w * KBD + kb) * 64 + lane) * KPL);
            frag fq = *reinterpret_cast<const frag *>(rec + Rec<D>::QP + ((w * KBD + kb) * 64 + lane) * KPL);
            u = M::mma(fw, sB[kb], u);
            o = M::mma(fq, sB[kb], o);
        }
        // publish U (elements e = 4 w + ii)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) ux[4 * w + ii] = (T)u[ii];
        __syncthreads();
        frag uB[KBC];
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb) uB[kb] = *reinterpret_cast<const frag *>(ux + kb * KPL);
        const float gc = a.gC[bh * a.NC + c];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            S[mt] *= gc;
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) {
                frag fd = *reinterpret_cast<const frag *>(
                    rec + Rec<D>::DKT + (((w * MT + mt) * KBC + kb) * 64 + lane) * KPL);
                S[mt] = M::mma(fd, uB[kb], S[mt]);
            }
        }
        // unnormalised output and its partial sum of squares over these 16 channels
        const int s0 = c * 64 + 16 * w + 4 * g;
        float *orow = a.ows + (bh * (size_t)a.NC * 64 + s0) * D + vcol;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            orow[(size_t)ii * D] = o[ii];
            float ss = o[ii] * o[ii];
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m, 64);
            if (n == ii) a.ps[(bh * NV + vb) * (size_t)a.NC * 64 + s0 + ii] = ss;
        }
    }
    if (a.S_T) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            *reinterpret_cast<floatx4 *>(a.S_T + (bh * D + vcol) * D + w * (D / 4) + 16 * mt + 4 * g) = S[mt];
    }
}

// ====================================================================== norm
template <class T, int D>
__global__ __launch_bounds__(kThreads) void gdn_norm_kernel(NormArgs a) {
    constexpr int G = D / 8;
    constexpr int NV = D / 16;
    const int tid = threadIdx.x, cg = tid % G;
    const int t = blockIdx.x * (kThreads / G) + tid / G;  // input (output) token
    const int h = blockIdx.y, b = blockIdx.z;
    if (t >= a.T) return;
    const size_t bh = (size_t)b * a.H + h;
    const size_t L = (size_t)a.NC * 64;
    float wv[8], gv[8], y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[i] = a.norm_w ? a.norm_w[h * D + 8 * cg + i] : 1.f;
    load8(static_cast<const T *>(a.gate) + (((size_t)b * a.T + t) * a.H + h) * D + 8 * cg, gv);
#pragma unroll
    for (int i = 0; i < 8; ++i) { gv[i] = wv[i] * silu(gv[i]); y[i] = 0.f; }
    for (int pass = 0; pass < (a.ows2 ? 2 : 1); ++pass) {
        const bool rev = pass == 0 ? a.reverse != 0 : true;
        const float *ows = pass == 0 ? a.ows : a.ows2;
        const float *ps = pass == 0 ? a.ps : a.ps2;
        const int s = rev ? a.T - 1 - t : t;  // scan position of this token
        float ss = 0.f;
#pragma unroll
        for (int vb = 0; vb < NV; ++vb) ss += ps[(bh * NV + vb) * L + s];
        const float inv = 1.0f / sqrtf(ss / D + a.eps);
        float ov[8];
        load8(ows + (bh * L + s) * D + 8 * cg, ov);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] += ov[i] * inv * gv[i];
    }
    store8(static_cast<T *>(a.out) + (((size_t)b * a.T + t) * a.H + h) * D + 8 * cg, y);
}

}  // namespace gdn

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
};

struct NormArgs {
    int B, T, H, NC, reverse;
    const float *ows;           // first (or only) scan
    const float *ows2;          // time-reversed scan, or null
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

// Short conv + SiLU (+ L2 normalisation for q and k) of the chunk's 64 scan
// positions into LDS.  Thread layout: G = D/8 threads per token row (8
// channels each); each thread owns RUN consecutive tokens and loads its
// RUN + 3 input rows (3 rows of causal history) once, all loads issued before
// any is used.
template <class T, int D>
__device__ __forceinline__ void prologue(const PrepArgs &a, PrepSmem<T, D> &sm, int c, int h, int b) {
    constexpr int G = D / 8;
    constexpr int RUN = 64 / (kThreads / G);
    constexpr int ROWS = RUN + 3;
    constexpr int LDX = PrepSmem<T, D>::LDX;
    const int tid = threadIdx.x, cg = tid % G, run = tid / G;
    const int s0 = c * 64 + run * RUN;
    const T *src[3] = {static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v)};
    const float *wsrc[3] = {a.conv_q, a.conv_k, a.conv_v};
    T *dst[3] = {sm.Qs, sm.Ks, sm.Vs};
    Raw8<T> raw[3][ROWS];
    bool rv[ROWS];
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) {
        const int sp = s0 - 3 + rr;
        rv[rr] = sp >= 0 && sp < a.T;
        int si = a.reverse ? a.T - 1 - sp : sp;
        si = si < 0 ? 0 : (si >= a.T ? a.T - 1 : si);
        const size_t off = (((size_t)b * a.T + si) * a.H + h) * D + 8 * cg;
#pragma unroll
        for (int x = 0; x < 3; ++x) raw[x][rr].load(src[x] + off);
    }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        float wt[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 wv = reinterpret_cast<const float4 *>(wsrc[x])[(size_t)h * D + 8 * cg + i];
            wt[i][0] = wv.x; wt[i][1] = wv.y; wt[i][2] = wv.z; wt[i][3] = wv.w;
        }
#pragma unroll
        for (int r = 0; r < RUN; ++r) {
            const bool valid = s0 + r < a.T;
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) s += rv[r + j] ? wt[i][j] * raw[x][r + j].get(i) : 0.f;
                acc[i] = valid ? silu(s) : 0.f;
            }
            if (x < 2) {
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) ss += acc[i] * acc[i];
#pragma unroll
                for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
                const float inv = valid ? 1.0f / sqrtf(ss + a.eps_l2) : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= inv;
            }
            T *row = dst[x] + (run * RUN + r) * LDX + 8 * cg;
#pragma unroll
            for (int i = 0; i < 8; ++i) row[i] = (T)acc[i];
        }
    }
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

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, n = lane % 16, g = lane / 16;

    // ---- gates: b and the cumulative log decay g inside the chunk
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
        sm.eg[tid] = expf(la);
        sm.dk[tid] = expf(__shfl(la, 63, 64) - la);
    }
    prologue<T, D>(a, sm, c, h, b);
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
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * w + 4 * g + ii, j = 16 * t + n;
                sm.Am[i * SM::LDA + j] = (j < i) ? sm.b[i] * expf(sm.g[i] - sm.g[j]) * acc[t][ii] : 0.f;
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
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int col = (D / 2) * w + 16 * ct + n;
            floatx4 acc;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int t = 16 * I + 4 * g + ii;
                acc[ii] = col < D ? sm.b[t] * sm.eg[t] * to_f(sm.Ks[t * SM::LDX + col])
                                  : sm.b[t] * to_f(sm.Vs[t * SM::LDX + col - D]);
            }
#pragma unroll
            for (int J = 0; J < I; ++J) acc = K::mma(aIJ[J], Xf[J][ct], acc);
            X[I][ct] = K::mma(tI, K::from4(acc), zero4());
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
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * w + 4 * g + ii, j = 16 * t + n;
                P[i * SM::LDP + j] = (T)((j <= i) ? expf(sm.g[i] - sm.g[j]) * acc[t][ii] : 0.f);
            }
        }
    }
    __syncthreads();

    // ---- P X on this wave's columns: Q' = e^g Q - P W (W columns), O0 = P U~
    T *rec = static_cast<T *>(a.rec) + (((size_t)b * a.H + h) * a.NC + c) * (size_t)Rec<D>::SIZE;
    {
        const T *P = sm.P();
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            frag pf[KBC];
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) pf[kb] = row_frag(P + (16 * R + n) * SM::LDP, kb, g);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = (D / 2) * w + 16 * ct + n;
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
                if (col < D) {
                    // Q' rows 16R + 4g + ii, staged in Qs over the q^ values it replaces
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int t = 16 * R + 4 * g + ii;
                        const float qv = sm.eg[t] * to_f(sm.Qs[t * SM::LDX + col]) - acc[ii];
                        sm.Qs[t * SM::LDX + col] = (T)qv;
                    }
                } else {
                    const int vb = (col - D) / 16;
                    store4(rec + Rec<D>::O0 + ((vb * 4 + R) * 64 + lane) * 4, acc);
                    store4(rec + Rec<D>::UT + ((vb * 4 + R) * 64 + lane) * 4, X[R][ct]);
                }
            }
        }
        // -W staged row-major in Vs (v^ is no longer needed)
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = (D / 2) * w + 16 * ct + n;
                if (col < D) {
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) sm.Vs[(16 * I + 4 * g + ii) * SM::LDX + col] = (T)(-X[I][ct][ii]);
                }
            }
    }
    __syncthreads();

    // ---- QP and WN as A fragments: rows = tokens 16w + n, K = key channels (chained)
    {
        const T *qrow = sm.Qs + (16 * w + n) * SM::LDX;
        const T *wrow = sm.Vs + (16 * w + n) * SM::LDX;
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            *reinterpret_cast<frag *>(rec + Rec<D>::QP + ((w * KBD + kb) * 64 + lane) * KPL) = row_frag(qrow, kb, g);
            *reinterpret_cast<frag *>(rec + Rec<D>::WN + ((w * KBD + kb) * 64 + lane) * KPL) = row_frag(wrow, kb, g);
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
    if (tid == 0) a.gC[((size_t)b * a.H + h) * a.NC + c] = sm.eg[63];
}

// ===================================================================== state
template <class T, int D> struct StateSmem {
    static constexpr int LDS_S = D / 4 + (sizeof(T) == 2 ? 8 : 4);
    static constexpr int LDS_U = 16 + (sizeof(T) == 2 ? 8 : 4);
    T Sx[64 * LDS_S];  // S^T as B fragments, per lane
    T Ux[64 * LDS_U];  // U as B fragments, per lane
};

// One chunk's operands for one wave of a state workgroup, in registers.
template <class T, int D> struct ChunkOps {
    typedef typename Mfma<T>::frag frag;
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int KBD = D / (4 * KPL);
    static constexpr int KBC = 16 / KPL;
    static constexpr int MT = D / 64;
    frag wn[KBD], qp[KBD], dk[MT][KBC];
    floatx4 ut, o0;
    float gc;
    __device__ __forceinline__ void load(const T *rec, const float *gcp, int vb, int w, int lane) {
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            wn[kb] = *reinterpret_cast<const frag *>(rec + Rec<D>::WN + ((w * KBD + kb) * 64 + lane) * KPL);
            qp[kb] = *reinterpret_cast<const frag *>(rec + Rec<D>::QP + ((w * KBD + kb) * 64 + lane) * KPL);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb)
                dk[mt][kb] = *reinterpret_cast<const frag *>(
                    rec + Rec<D>::DKT + (((w * MT + mt) * KBC + kb) * 64 + lane) * KPL);
        ut = load4(rec + Rec<D>::UT + ((vb * 4 + w) * 64 + lane) * 4);
        o0 = load4(rec + Rec<D>::O0 + ((vb * 4 + w) * 64 + lane) * 4);
        gc = *gcp;
    }
};

// Workgroup placement: launched as a 1-D grid whose size is a multiple of 8.
// Consecutive workgroup ids go to different XCDs (round robin), so id L is
// mapped to position p = (L % 8) * per + L / 8 of the head-major list of
// (batch*head, value block) pairs: the value blocks of one head then sit on
// one XCD (two at most) and share its L2 for the head's chunk records.
__device__ __forceinline__ bool xcd_position(int L, int nwg_used, int nwg_launched, int &p) {
    const int per = nwg_launched / 8;
    p = (L % 8) * per + L / 8;
    return p < nwg_used;
}

// One workgroup owns a block of 16 value channels of one head.  Wave w
// computes U and O for tokens 16w..16w+15 (K = all key channels) and updates
// the key-channel rows w*D/4.. of S^T (K = all tokens); S^T and U are
// exchanged through LDS once per chunk each.
template <class T, int D>
__global__ __launch_bounds__(kThreads) void gdn_state_kernel(StateArgs a) {
    typedef Mfma<T> M;
    typedef typename M::frag frag;
    typedef ChunkOps<T, D> Ops;
    constexpr int KPL = M::KPL;
    constexpr int KBD = Ops::KBD;
    constexpr int KBC = Ops::KBC;
    constexpr int MT = Ops::MT;
    constexpr int NV = D / 16;
    typedef StateSmem<T, D> SM;
    __shared__ SM sm;

    int p;
    if (!xcd_position(blockIdx.x, a.B * a.H * NV, gridDim.x, p)) return;
    const int vb = p % NV;
    const size_t bh = p / NV;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, n = lane % 16, g = lane / 16;
    const int vcol = 16 * vb + n;

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
    const float *gc0 = a.gC + bh * a.NC;
    T *sx = sm.Sx + lane * SM::LDS_S;
    T *ux = sm.Ux + lane * SM::LDS_U;

    auto step = [&](const Ops &f, int c) {
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
        floatx4 u = f.ut, o = f.o0;
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
            u = M::mma(f.wn[kb], sB[kb], u);
            o = M::mma(f.qp[kb], sB[kb], o);
        }
        // publish U (elements e = 4 w + ii)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) ux[4 * w + ii] = (T)u[ii];
        __syncthreads();
        frag uB[KBC];
#pragma unroll
        for (int kb = 0; kb < KBC; ++kb) uB[kb] = *reinterpret_cast<const frag *>(ux + kb * KPL);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            S[mt] *= f.gc;
#pragma unroll
            for (int kb = 0; kb < KBC; ++kb) S[mt] = M::mma(f.dk[mt][kb], uB[kb], S[mt]);
        }
        // unnormalised output (the normalisation pass reduces over all channels)
        const int s0 = c * 64 + 16 * w + 4 * g;
        float *orow = a.ows + (bh * (size_t)a.NC * 64 + s0) * D + vcol;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) orow[(size_t)ii * D] = o[ii];
    };

    // two register sets: chunk c+1's operands load while chunk c computes.  The
    // loads are unconditional (the index is clamped to the last chunk) and the
    // loop has no early exit, so no branch merges different loads in flight.
    Ops A, B;
    const int last = a.NC - 1;
    auto at = [&](int cc) { return rec0 + (size_t)min(cc, last) * Rec<D>::SIZE; };
    auto gat = [&](int cc) { return gc0 + min(cc, last); };
    A.load(at(0), gat(0), vb, w, lane);
    const int pairs = a.NC / 2;
    for (int i = 0; i < pairs; ++i) {
        const int c = 2 * i;
        B.load(at(c + 1), gat(c + 1), vb, w, lane);
        step(A, c);
        A.load(at(c + 2), gat(c + 2), vb, w, lane);
        step(B, c + 1);
    }
    if (a.NC & 1) step(A, a.NC - 1);
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
    const int tid = threadIdx.x, cg = tid % G;
    const int t0 = blockIdx.x * (kThreads / G) + tid / G;  // input (output) token
    const bool live = t0 < a.T;
    const int t = live ? t0 : a.T - 1;  // idle threads still take part in the shuffles
    const int h = blockIdx.y, b = blockIdx.z;
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
        const int s = rev ? a.T - 1 - t : t;  // scan position of this token
        float ov[8];
        load8(ows + (bh * L + s) * D + 8 * cg, ov);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += ov[i] * ov[i];
#pragma unroll
        for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float inv = 1.0f / sqrtf(ss / D + a.eps);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] += ov[i] * inv * gv[i];
    }
    if (live) store8(static_cast<T *>(a.out) + (((size_t)b * a.T + t) * a.H + h) * D + 8 * cg, y);
}

}  // namespace gdn

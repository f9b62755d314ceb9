// bwd.hpp -- gfx950 kernels of the GDN layer's backward pass: the gradients
// of the layer forward (short conv + SiLU, L2-normalised q and k, the gated
// delta rule in 64-token chunks, the gated RMS normalisation) with respect to
// every input.
//
// The backward follows the forward's chunking: the chunked WY form, which
// comes from unrolling the gated delta rule inside a 64-token chunk.  (The
// LinMorph project page, "Abstract", trains the converted GDN blocks by
// progressive distillation and joint recovery, which needs these gradients.)
// For chunk c with entry state S
// (value rows, key columns), tokens as rows, g the cumulative log decay
// inside the chunk, gam = e^g, gC = e^{g_last}, dl = e^{g_last - g}:
//   A = strictly lower (b_i e^{g_i - g_j} k_i . k_j),  T = (I + A)^-1
//   W = T diag(b gam) K,  U~ = T diag(b) V,  U = U~ - W S^T
//   P = lower-inclusive (e^{g_i - g_j} q_i . k_j),  Q' = diag(gam) Q - P W
//   O = Q' S^T + P U~,  S_next = gC S + U^T diag(dl) K
// Given dO and dS_next, the entry-state gradient runs backwards over chunks,
//   dS = gC dS_next - (dS_next (diag(dl) K)^T) W + dO^T Q',
// and every other gradient of the chunk follows from S, dS_next and dO alone
// (kernel bwd_grad_kernel lists the steps).
//
// Everything is fp32, on v_mfma_f32_16x16x4_f32.  The chunk quantities live
// in the workspace as row-major fp32 arrays, one record per (batch row,
// head, chunk).  Kernels, in launch order:
//   bwd_prep_kernel      per chunk (8 waves): recomputed q^, k^, v^; A, T, W, U~, P, Q', D K
//   bwd_state_kernel     per 16 value rows: the forward chain, entry states
//   bwd_out_kernel       per chunk: O, then the gated RMS norm's backward (dO, dgate)
//   bwd_dstate_kernel    per 16 value rows: the entry-state gradients, last chunk first
//   bwd_grad_kernel      per chunk: dq^, dk^, dv^, d log a, db
//   bwd_prologue_kernel  per chunk: L2 norm, SiLU and conv backward: dq, dk,
//                        dv, conv-weight partial sums
//   bwd_reduce_kernel    the conv-weight and norm-weight sums
#pragma once
#include "frag.hpp"
#include "sync.hpp"

namespace gdnb {

using gdn::bf16;
using gdn::floatx4;

constexpr int C = 64;     // tokens per chunk
constexpr int NT = 256;   // threads per workgroup (4 waves)
constexpr int GW = 8, GNT = 64 * GW;  // waves and threads of bwd_prep_kernel and bwd_grad_kernel

// Offsets (in floats) inside one chunk record; all row-major.
template <int D> struct Rec {
    static constexpr int XQ = 0;             // q^  [64][D]
    static constexpr int XK = 64 * D;        // k^
    static constexpr int XV = 128 * D;       // v^
    static constexpr int W = 192 * D;        // W
    static constexpr int UT = 256 * D;       // U~
    static constexpr int QP = 320 * D;       // Q'
    static constexpr int DK = 384 * D;       // diag(dl) K
    static constexpr int DO = 448 * D;       // dO
    static constexpr int DXQ = 512 * D;      // dq^
    static constexpr int DXK = 576 * D;      // dk^
    static constexpr int DXV = 640 * D;      // dv^
    static constexpr int TM = 704 * D;       // T [64][64]
    static constexpr int P = TM + 64 * 64;   // P [64][64]
    static constexpr int G = P + 64 * 64;    // g [64], then gC
    static constexpr int SC = G + 128;       // entry state S [D][D]
    static constexpr int DSN = SC + D * D;   // gradient of the exit state [D][D]
    static constexpr int WT = DSN + D * D;   // W, key-major [D][64]
    static constexpr int DKT = WT + 64 * D;  // D K, key-major
    static constexpr int QPT = DKT + 64 * D; // Q', key-major
    static constexpr int EKK = QPT + 64 * D; // strictly lower e^{g_i - g_j} k_i . k_j [64][64]
    static constexpr int SIZE = EKK + 64 * 64;
};

struct Args {
    int B, T, H, NC;
    int c0, c1;                                        // this launch's chunks: c0 .. c1 - 1
    const void *q, *k, *v, *gate, *dy;                 // [B, T, H, D], I/O dtype
    const float *log_a, *beta;                         // [B, T, H]
    const float *conv_q, *conv_k, *conv_v;             // [H D, 4]
    const float *norm_w;                               // [H, D] or null (ones)
    const float *S0, *dS_T;                            // [B, H, D, D] or null (zero)
    float eps_l2, eps_norm;
    void *dq, *dk, *dv, *dgate;                        // [B, T, H, D], I/O dtype
    float *dlog_a, *dbeta;                             // [B, T, H]
    float *dconv_q, *dconv_k, *dconv_v;                // [H D, 4]
    float *dnorm_w;                                    // [H, D] or null
    float *dS0;                                        // [B, H, D, D] or null
    float *rec;                                        // B H NC chunk records
    float *part_conv;                                  // [B NC H][3][D][4]
    float *part_norm;                                  // [B NC H][D]
    float *sink;                                       // [B, H, D, D]: the chains' stores past either end
    int reverse;                                       // 1: the layer on the time-reversed sequence
    const int *cu;                                     // variable lengths: B + 1 row offsets, or null
};

// Sequence b: its first token row and its length.  Without a table, row b of
// a [B, T] batch; with one, rows cu[b] .. cu[b+1] - 1 of the packed tokens
// (T is then the longest length, and every sequence has NC chunk records).
struct Seq {
    long long off;
    int len;
};
__device__ __forceinline__ Seq seq_of(const Args &a, int b) {
    if (a.cu) return Seq{a.cu[b], a.cu[b + 1] - a.cu[b]};
    return Seq{(long long)b * a.T, a.T};
}
// Input / output row (within the sequence) of scan position t; the records
// are in scan order.
__device__ __forceinline__ int src_t(const Args &a, const Seq &q, int t) { return a.reverse ? q.len - 1 - t : t; }

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float silu(float x) { return x * sigm(x); }
__device__ __forceinline__ float dsilu(float x) {
    const float s = sigm(x);
    return s * (1.0f + x * (1.0f - s));
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// One 16 x 16 tile of acc + A B, A rows m0.. (16 x K), B columns n0.. (K x 16),
// fp32 MFMA 16x16x4.  Lane (r, g) (r = lane % 16, g = lane / 16) supplies
// k = k0 + 4 g + j to the j-th product of each 16-deep step, for A and B
// alike, so the 4 products sum all 16 k.
//   KA: A(m, k) at A[m lda + k] (k contiguous, read 4 at a time), else A[k lda + m]
//   KB: B(k, n) at B[n ldb + k] (k contiguous), else B[k ldb + n]
// acc[i] is the element (m0 + 4 g + i, n0 + r).
template <bool KA, bool KB, int K>
__device__ __forceinline__ floatx4 mm16(floatx4 acc, const float *A, int lda, int m0, const float *B, int ldb,
                                        int n0) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll 4
    for (int k0 = 0; k0 < K; k0 += 16) {
        float a[4], b[4];
        if constexpr (KA) {
            const float4 t = *reinterpret_cast<const float4 *>(A + (size_t)(m0 + r) * lda + k0 + 4 * g);
            a[0] = t.x; a[1] = t.y; a[2] = t.z; a[3] = t.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = A[(size_t)(k0 + 4 * g + j) * lda + m0 + r];
        }
        if constexpr (KB) {
            const float4 t = *reinterpret_cast<const float4 *>(B + (size_t)(n0 + r) * ldb + k0 + 4 * g);
            b[0] = t.x; b[1] = t.y; b[2] = t.z; b[3] = t.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = B[(size_t)(k0 + 4 * g + j) * ldb + n0 + r];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
    }
    return acc;
}

__device__ __forceinline__ floatx4 z4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// The A operand of mm16 held in registers, for a wave that multiplies the
// same 16 rows by several column tiles: af[step][j] is what lane (r, g)
// supplies to product j of 16-deep step `step`.
template <bool KA, int K>
__device__ __forceinline__ void load_a(float (&af)[K / 16][4], const float *A, int lda, int m0) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < K / 16; ++ks) {
        if constexpr (KA) {
            const floatx4 t = *reinterpret_cast<const floatx4 *>(A + (size_t)(m0 + r) * lda + 16 * ks + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) af[ks][j] = t[j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) af[ks][j] = A[(size_t)(16 * ks + 4 * g + j) * lda + m0 + r];
        }
    }
}
template <bool KB, int K>
__device__ __forceinline__ floatx4 mm16a(floatx4 acc, const float (&af)[K / 16][4], const float *B, int ldb, int n0) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < K / 16; ++ks) {
        float b[4];
        if constexpr (KB) {
            const floatx4 t = *reinterpret_cast<const floatx4 *>(B + (size_t)(n0 + r) * ldb + 16 * ks + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = t[j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = B[(size_t)(16 * ks + 4 * g + j) * ldb + n0 + r];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[ks][j], b[j], acc, 0, 0, 0);
    }
    return acc;
}

// 8 consecutive channels of one token row, loaded with one (bf16) or two
// (fp32) 16-byte loads; a row outside the sequence reads as zeros.
template <class IO> struct Row8;
template <> struct Row8<bf16> {
    uint4 u;
    __device__ __forceinline__ void load(const bf16 *p, bool ok) {
        u = ok ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
    }
    __device__ __forceinline__ float get(int i) const {
        const unsigned w = (&u.x)[i >> 1];
        return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};
template <> struct Row8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p, bool ok) {
        a = ok ? *reinterpret_cast<const float4 *>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
        b = ok ? *reinterpret_cast<const float4 *>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __device__ __forceinline__ float get(int i) const { return i < 4 ? (&a.x)[i] : (&b.x)[i - 4]; }
};

template <int D> __device__ __forceinline__ float *record(const Args &a, int b, int h, int c) {
    return a.rec + (((size_t)b * a.H + h) * a.NC + c) * (size_t)Rec<D>::SIZE;
}

// ---------------------------------------------------------------------------
// Per chunk: q^, k^, v^ (short conv, SiLU, L2 norms, recomputed from the
// inputs), the gates, A, T = (I + A)^-1, W, U~, P, Q' and D K.  Tokens past
// the sequence's end are zero rows with b = 0 and log a = 0, which leave the
// state and every gradient unchanged.
template <class IO, int D>
__global__ __launch_bounds__(GNT) void bwd_prep_kernel(Args a) {
    typedef Rec<D> R;
    constexpr int LX = D + 4, LC = C + 4;
    extern __shared__ __align__(16) float lds[];
    float *sQ = lds, *sK = sQ + C * LX, *sV = sK + C * LX, *sT = sV + C * LX, *sM = sT + C * LC;
    float *sg = sM + C * LC, *sb = sg + C, *sgam = sb + C, *sTmp = sgam + C;
    const int c = a.c0 + blockIdx.x, h = blockIdx.y, b = blockIdx.z, t0 = c * C;
    // 8 waves: wave w takes row block rb (16 tokens) and the column tiles hf, hf + 2, ...
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, r = lane % 16, g = lane / 16;
    const int rb = w % 4, hf = w / 4;
    float *rec = record<D>(a, b, h, c);
    const Seq sq = seq_of(a, b);

    if (tid < 64) {
        const int t = t0 + tid;
        const bool valid = t < sq.len;
        const int ts = valid ? src_t(a, sq, t) : 0;
        float la = valid ? a.log_a[((size_t)sq.off + ts) * a.H + h] : 0.f;
        const float be = valid ? a.beta[((size_t)sq.off + ts) * a.H + h] : 0.f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(la, o, 64);
            if (tid >= o) la += y;
        }
        sg[tid] = la;
        sb[tid] = be;
        sgam[tid] = expf(la);
        rec[R::G + tid] = la;
        if (tid == 63) rec[R::G + 64] = expf(la);
    }
    // short conv + SiLU of q, k, v (tap j multiplies x_{t-3+j}; zeros before the
    // start), L2 norms of q and k.  Thread: 8 channels (one 16- or 32-byte load per row) of RUN
    // consecutive tokens; its RUN + 3 input rows of q, k and v are all loaded
    // before any arithmetic.
    {
        constexpr int G = D / 8, RUN = 64 / (GNT / G), ROWS = RUN + 3;
        const int cg = tid % G, run = tid / G, s0 = t0 + run * RUN;
        const IO *src[3] = {static_cast<const IO *>(a.q), static_cast<const IO *>(a.k), static_cast<const IO *>(a.v)};
        const float *cw[3] = {a.conv_q, a.conv_k, a.conv_v};
        float *dst[3] = {sQ, sK, sV};
        Row8<IO> raw[3][ROWS];
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr) {
            const int sp = s0 - 3 + rr;
            const bool ok = sp >= 0 && sp < sq.len;
            const size_t off = ((((size_t)sq.off + (ok ? src_t(a, sq, sp) : 0)) * a.H + h) * D) + 8 * cg;
#pragma unroll
            for (int x = 0; x < 3; ++x) raw[x][rr].load(src[x] + off, ok);
        }
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            float wt[8][4];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 wv = *reinterpret_cast<const float4 *>(cw[x] + ((size_t)h * D + 8 * cg + i) * 4);
                wt[i][0] = wv.x; wt[i][1] = wv.y; wt[i][2] = wv.z; wt[i][3] = wv.w;
            }
#pragma unroll
            for (int rt = 0; rt < RUN; ++rt) {
                const bool valid = s0 + rt < sq.len;
                float out[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float z = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) z = fmaf(wt[i][j], raw[x][rt + j].get(i), z);
                    out[i] = valid ? silu(z) : 0.f;
                }
                if (x < 2) {
                    // L2 norm of the token's row: its D channels sit on the G
                    // neighbouring lanes of this run
                    float ss = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) ss += out[i] * out[i];
                    const float rho = 1.0f / sqrtf(gdn::group_sum<G>(ss) + a.eps_l2);
#pragma unroll
                    for (int i = 0; i < 8; ++i) out[i] *= rho;
                }
                float *row = dst[x] + (run * RUN + rt) * LX + 8 * cg;
                *reinterpret_cast<float4 *>(row) = make_float4(out[0], out[1], out[2], out[3]);
                *reinterpret_cast<float4 *>(row + 4) = make_float4(out[4], out[5], out[6], out[7]);
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < C * D / 4; idx += GNT) {
        const int tl = idx / (D / 4), c4 = 4 * (idx % (D / 4));
        *reinterpret_cast<float4 *>(rec + R::XQ + tl * D + c4) = *reinterpret_cast<const float4 *>(sQ + tl * LX + c4);
        *reinterpret_cast<float4 *>(rec + R::XK + tl * D + c4) = *reinterpret_cast<const float4 *>(sK + tl * LX + c4);
        *reinterpret_cast<float4 *>(rec + R::XV + tl * D + c4) = *reinterpret_cast<const float4 *>(sV + tl * LX + c4);
    }
    // A = strictly lower (b_i e^{g_i - g_j} k_i . k_j)
    for (int j = 0; j < 2; ++j) {
        const int nt = 2 * j + hf;
        floatx4 acc = z4();
        if (nt <= rb) acc = mm16<true, true, D>(acc, sK, LX, 16 * rb, sK, LX, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i, col = 16 * nt + r;
            const float ekk = col < row ? expf(sg[row] - sg[col]) * acc[i] : 0.f;
            sM[row * LC + col] = sb[row] * ekk;
            rec[R::EKK + row * C + col] = ekk;
        }
    }
    __syncthreads();
    // T = (I + A)^-1 in 16 x 16 blocks.  Diagonal blocks: wave w inverts
    // (I + A_ww) by forward substitution, column n on lane n (lanes 0..15);
    // the blocks above the diagonal are zero.
    if (w < 4)
        for (int idx = lane; idx < 16 * 64; idx += 64) {
            const int i = 16 * w + idx / 64, j = idx % 64;
            if (j < 16 * w || j >= 16 * w + 16) sT[i * LC + j] = 0.f;
        }
    if (w < 4 && lane < 16) {
        const int n = lane;
        const float *Aw = sM + 16 * w * LC + 16 * w;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) s = fmaf(Aw[i * LC + m], x[m], s);
            x[i] = i < n ? 0.f : (i == n ? 1.f : -s);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(16 * w + i) * LC + 16 * w + n] = x[i];
    }
    __syncthreads();
    // Blocks below the diagonal, block row by block row:
    //   T_IJ = -T_II (sum_{J <= K < I} A_IK T_KJ),  wave J computes T_IJ
    float *tmp = sTmp + w * 16 * 20;
    for (int I = 1; I < 4; ++I) {
        if (w < I) {
            floatx4 acc = z4();
            for (int K = w; K < I; ++K)
                acc = mm16<true, false, 16>(acc, sM + 16 * I * LC + 16 * K, LC, 0, sT + 16 * K * LC + 16 * w, LC, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) tmp[(4 * g + i) * 20 + r] = acc[i];
        }
        __syncthreads();
        if (w < I) {
            const floatx4 t = mm16<true, false, 16>(z4(), sT + 16 * I * LC + 16 * I, LC, 0, tmp, 20, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(16 * I + 4 * g + i) * LC + 16 * w + r] = -t[i];
        }
        __syncthreads();
    }
    // T out; T' = T diag(b gam) into the A storage; diag(b) V in place
    for (int idx = tid; idx < C * C; idx += GNT) {
        const int i = idx / C, j = idx % C;
        const float t = sT[i * LC + j];
        rec[R::TM + idx] = t;
        sM[i * LC + j] = t * sb[j] * sgam[j];
    }
    for (int idx = tid; idx < C * D; idx += GNT) {
        const int tl = idx / D, ch = idx % D;
        sV[tl * LX + ch] *= sb[tl];
    }
    __syncthreads();
    // U~ = T diag(b) V
    for (int j = 0; j < D / 32; ++j) {
        const int nt = 2 * j + hf;
        const floatx4 acc = mm16<true, false, C>(z4(), sT, LC, 16 * rb, sV, LX, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) rec[R::UT + (16 * rb + 4 * g + i) * D + 16 * nt + r] = acc[i];
    }
    __syncthreads();
    // W = T diag(b gam) K, out and into the V storage
    for (int j = 0; j < D / 32; ++j) {
        const int nt = 2 * j + hf;
        const floatx4 acc = mm16<true, false, C>(z4(), sM, LC, 16 * rb, sK, LX, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i, col = 16 * nt + r;
            rec[R::W + row * D + col] = acc[i];
            sV[row * LX + col] = acc[i];
        }
    }
    __syncthreads();
    // P = lower-inclusive (e^{g_i - g_j} q_i . k_j), out and into the A storage
    for (int j = 0; j < 2; ++j) {
        const int nt = 2 * j + hf;
        floatx4 acc = z4();
        if (nt <= rb) acc = mm16<true, true, D>(acc, sQ, LX, 16 * rb, sK, LX, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i, col = 16 * nt + r;
            const float p = col <= row ? expf(sg[row] - sg[col]) * acc[i] : 0.f;
            sM[row * LC + col] = p;
            rec[R::P + row * C + col] = p;
        }
    }
    __syncthreads();
    // Q' = diag(gam) Q - P W;  D K = diag(e^{g_last - g}) K
    for (int j = 0; j < D / 32; ++j) {
        const int nt = 2 * j + hf;
        const floatx4 acc = mm16<true, false, C>(z4(), sM, LC, 16 * rb, sV, LX, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i, col = 16 * nt + r;
            const float qp = sgam[row] * sQ[row * LX + col] - acc[i];
            rec[R::QP + row * D + col] = qp;
            sQ[row * LX + col] = qp;
        }
    }
    const float glast = sg[63];
    for (int idx = tid; idx < C * D; idx += GNT) {
        const int tl = idx / D, ch = idx % D;
        rec[R::DK + idx] = expf(glast - sg[tl]) * sK[tl * LX + ch];
    }
    __syncthreads();
    // key-major copies of W, D K and Q' (the chains read them as B operands)
    for (int idx = tid; idx < C * D; idx += GNT) {
        const int key = idx / C, tl = idx % C;
        rec[R::WT + idx] = sV[tl * LX + key];
        rec[R::DKT + idx] = expf(glast - sg[tl]) * sK[tl * LX + key];
        rec[R::QPT + idx] = sQ[tl * LX + key];
    }
}

// ---------------------------------------------------------------------------
// The chains.  A workgroup owns 16 value rows of one head's state (4 waves);
// each wave loads its own MFMA operands of a chunk straight into registers,
// one chunk ahead (two register sets used in turn), so that a step waits for
// no memory.  The items of a head are neighbours in the work list and share
// one XCD's L2 (the 8 workgroups of a head read the same W and D K).
template <int D> struct FwdOps {
    static constexpr int KS = D / 16, NTW = D / 64;
    floatx4 wa[KS];         // W rows 16 w + r, keys 16 ks + 4 g ..: A of W S^T
    floatx4 kb[NTW][4];     // (D K)^T rows 16 nt + r (nt = w + 4 j), tokens 16 ks + 4 g ..: B of U^T D K
    float ut[4];            // U~ (token 16 w + 4 g + i, value 16 vb + r)
    float gC;
};

template <int D>
__device__ __forceinline__ void fwd_ops_load(FwdOps<D> &o, const float *rc, int vb) {
    typedef Rec<D> R;
    const int w = threadIdx.x / 64, lane = threadIdx.x % 64, r = lane % 16, g = lane / 16;
#pragma unroll
    for (int ks = 0; ks < FwdOps<D>::KS; ++ks)
        o.wa[ks] = *reinterpret_cast<const floatx4 *>(rc + R::W + (16 * w + r) * D + 16 * ks + 4 * g);
#pragma unroll
    for (int j = 0; j < FwdOps<D>::NTW; ++j)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            o.kb[j][ks] = *reinterpret_cast<const floatx4 *>(rc + R::DKT + (16 * (w + 4 * j) + r) * C + 16 * ks + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) o.ut[i] = rc[R::UT + (16 * w + 4 * g + i) * D + 16 * vb + r];
    o.gC = rc[R::G + 64];
}

// The forward chain for value rows 16 vb .. of one head: each chunk's entry
// state goes to its record; U = U~ - W S^T (wave w: tokens 16 w ..), then
// S <- gC S + U^T D K (wave w: key tiles w, w + 4, ...).
template <int D>
__global__ __launch_bounds__(NT) void bwd_state_kernel(Args a) {
    typedef Rec<D> R;
    typedef FwdOps<D> O;
    constexpr int LS = D + 4, LU = 16 + 4;
    __shared__ __align__(16) float sS[16 * LS];
    __shared__ __align__(16) float sU[C * LU];
    constexpr int NV = D / 16;
    int pos;
    if (!gdn::xcd_position(blockIdx.x, a.B * a.H * NV, gridDim.x, pos)) return;
    const int vb = pos % NV, h = (pos / NV) % a.H, b = pos / NV / a.H;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, r = lane % 16, g = lane / 16;
    // the range's entry state: S0 for the first chunk, else what the previous
    // range stored as this chunk's entry state
    float *rec0 = record<D>(a, b, h, a.c0);
    for (int idx = tid; idx < 16 * D; idx += NT) {
        const int row = idx / D, col = idx % D;
        float *p = rec0 + R::SC + (16 * vb + row) * D + col;
        if (a.c0 == 0) {
            const float v = a.S0 ? a.S0[(((size_t)b * a.H + h) * D + 16 * vb + row) * D + col] : 0.f;
            sS[row * LS + col] = v;
            *p = v;
        } else {
            sS[row * LS + col] = *p;
        }
    }
    __syncthreads();

    auto step = [&](const O &o, int c) {
        // U = U~ - W S^T for tokens 16 w .. (B operand: S rows r, read k-contiguous)
        floatx4 acc = z4();
#pragma unroll
        for (int ks = 0; ks < O::KS; ++ks) {
            const floatx4 sv = *reinterpret_cast<const floatx4 *>(sS + r * LS + 16 * ks + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o.wa[ks][j], sv[j], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sU[(16 * w + 4 * g + i) * LU + r] = o.ut[i] - acc[i];
        gdn::lds_barrier();
        // S <- gC S + U^T D K on this wave's key tiles; the result is the next
        // chunk's entry state (after the last chunk: the sink).  Loads and
        // stores are unconditional so that the wait counts stay exact.
        float *rn = c + 1 < a.NC ? record<D>(a, b, h, c + 1) + R::SC : a.sink + ((size_t)b * a.H + h) * D * D;
#pragma unroll
        for (int j = 0; j < O::NTW; ++j) {
            const int nt = w + 4 * j;
            floatx4 s4;
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[i] = o.gC * sS[(4 * g + i) * LS + 16 * nt + r];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(sU[(16 * ks + 4 * g + jj) * LU + r], o.kb[j][ks][jj], s4,
                                                             0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sS[(4 * g + i) * LS + 16 * nt + r] = s4[i];
                rn[(16 * vb + 4 * g + i) * D + 16 * nt + r] = s4[i];
            }
        }
        gdn::lds_barrier();
    };

    O oa, ob;
    fwd_ops_load<D>(oa, rec0, vb);
    // (the scheduling barriers keep the next chunk's loads ahead of the step)
    for (int c = a.c0; c < a.c1; c += 2) {
        fwd_ops_load<D>(ob, record<D>(a, b, h, min(c + 1, a.c1 - 1)), vb);
        __builtin_amdgcn_sched_barrier(0);
        step(oa, c);
        if (c + 1 >= a.c1) break;
        fwd_ops_load<D>(oa, record<D>(a, b, h, min(c + 2, a.c1 - 1)), vb);
        __builtin_amdgcn_sched_barrier(0);
        step(ob, c + 1);
    }
}

// ---------------------------------------------------------------------------
// Per chunk: O = Q' S^T + P U~ (wave w: tokens 16w..), then the backward of
// y = O / sqrt(mean(O^2) + eps) * w * SiLU(gate): dO to the record, dgate
// out, and this chunk's part of the norm weight's gradient.
template <class IO, int D>
__global__ __launch_bounds__(NT) void bwd_out_kernel(Args a) {
    typedef Rec<D> R;
    constexpr int NTL = D / 16;
    __shared__ float sN[4][D];
    const int c = a.c0 + blockIdx.x, h = blockIdx.y, b = blockIdx.z, t0 = c * C;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, r = lane % 16, g = lane / 16;
    float *rec = record<D>(a, b, h, c);
    const Seq sq = seq_of(a, b);
    floatx4 o[NTL];
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
    float aq[D / 16][4], ap[C / 16][4];  // this wave's rows of Q' and P, used for every column tile
    load_a<true, D>(aq, rec + R::QP, D, 16 * w);
    load_a<true, C>(ap, rec + R::P, C, 16 * w);
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
        o[nt] = mm16a<true, D>(z4(), aq, rec + R::SC, D, 16 * nt);
        o[nt] = mm16a<false, C>(o[nt], ap, rec + R::UT, D, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) ss[i] += o[nt][i] * o[nt][i];
    }
    float rr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rr[i] = 1.0f / sqrtf(gdn::group_sum<16>(ss[i]) / D + a.eps_norm);
    const IO *gate = static_cast<const IO *>(a.gate);
    const IO *dy = static_cast<const IO *>(a.dy);
    IO *dgate = static_cast<IO *>(a.dgate);
    float gt[NTL][4], dyv[NTL][4], dot[4] = {0.f, 0.f, 0.f, 0.f}, cs[NTL];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
        const int col = 16 * nt + r;
        const float wn = a.norm_w ? a.norm_w[(size_t)h * D + col] : 1.f;
        cs[nt] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * w + 4 * g + i;
            const size_t off = (((size_t)sq.off + (t < sq.len ? src_t(a, sq, t) : 0)) * a.H + h) * D + col;
            gt[nt][i] = t < sq.len ? to_f(gate[off]) : 0.f;
            dyv[nt][i] = t < sq.len ? to_f(dy[off]) : 0.f;
            const float n = o[nt][i] * rr[i], sgt = silu(gt[nt][i]);
            dot[i] += dyv[nt][i] * wn * sgt * n;
            cs[nt] += dyv[nt][i] * n * sgt;
            if (t < sq.len) dgate[off] = (IO)(dyv[nt][i] * n * wn * dsilu(gt[nt][i]));
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dot[i] = gdn::group_sum<16>(dot[i]) / D;
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
        const int col = 16 * nt + r;
        const float wn = a.norm_w ? a.norm_w[(size_t)h * D + col] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * w + 4 * g + i;
            const float n = o[nt][i] * rr[i];
            const float dn = dyv[nt][i] * wn * silu(gt[nt][i]);
            rec[R::DO + row * D + col] = rr[i] * (dn - n * dot[i]);
        }
        // column sums over the wave's 16 rows: lanes r, r + 16, r + 32, r + 48
        float s = cs[nt];
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (g == 0) sN[w][col] = s;
    }
    __syncthreads();
    if (tid < D)
        a.part_norm[(((size_t)b * a.NC + c) * a.H + h) * D + tid] = sN[0][tid] + sN[1][tid] + sN[2][tid] + sN[3][tid];
}

// ---------------------------------------------------------------------------
// Operands of one reverse-chain step, per wave (see FwdOps).
template <int D> struct RevOps {
    static constexpr int KS = D / 16, NTW = D / 64;
    floatx4 ka[KS];         // D K rows 16 w + r (tokens), keys 16 ks + 4 g ..: B of dS (D K)^T
    floatx4 wb[NTW][4];     // W^T rows 16 nt + r (keys), tokens 16 ks + 4 g ..: B of X W
    floatx4 qb[NTW][4];     // Q'^T likewise: B of dO^T Q'
    float oa[4][4];         // dO (token 16 ks + 4 g + jj, value 16 vb + r): A of dO^T Q'
    float gC;
};

template <int D>
__device__ __forceinline__ void rev_ops_load(RevOps<D> &o, const float *rc, int vb) {
    typedef Rec<D> R;
    const int w = threadIdx.x / 64, lane = threadIdx.x % 64, r = lane % 16, g = lane / 16;
#pragma unroll
    for (int ks = 0; ks < RevOps<D>::KS; ++ks)
        o.ka[ks] = *reinterpret_cast<const floatx4 *>(rc + R::DK + (16 * w + r) * D + 16 * ks + 4 * g);
#pragma unroll
    for (int j = 0; j < RevOps<D>::NTW; ++j)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int off = (16 * (w + 4 * j) + r) * C + 16 * ks + 4 * g;
            o.wb[j][ks] = *reinterpret_cast<const floatx4 *>(rc + R::WT + off);
            o.qb[j][ks] = *reinterpret_cast<const floatx4 *>(rc + R::QPT + off);
        }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o.oa[ks][jj] = rc[R::DO + (16 * ks + 4 * g + jj) * D + 16 * vb + r];
    o.gC = rc[R::G + 64];
}

// Entry-state gradients for value rows 16 vb .. of one head, last chunk
// first.  Each chunk's exit-state gradient goes to its record; then
// dS <- gC dS - (dS (D K)^T) W + dO^T Q' (X = dS (D K)^T: wave w tokens 16 w ..;
// the update: wave w key tiles w, w + 4, ...).
template <int D>
__global__ __launch_bounds__(NT) void bwd_dstate_kernel(Args a) {
    typedef Rec<D> R;
    typedef RevOps<D> O;
    constexpr int LS = D + 4, LXX = C + 4;
    __shared__ __align__(16) float sD[16 * LS];
    __shared__ __align__(16) float sX[16 * LXX];
    constexpr int NV = D / 16;
    int pos;
    if (!gdn::xcd_position(blockIdx.x, a.B * a.H * NV, gridDim.x, pos)) return;
    const int vb = pos % NV, h = (pos / NV) % a.H, b = pos / NV / a.H;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, r = lane % 16, g = lane / 16;
    // the range's last chunk's exit-state gradient: dS_T for the sequence's last
    // chunk, else what the following range stored
    float *recl = record<D>(a, b, h, a.c1 - 1);
    for (int idx = tid; idx < 16 * D; idx += NT) {
        const int row = idx / D, col = idx % D;
        float *p = recl + R::DSN + (16 * vb + row) * D + col;
        if (a.c1 == a.NC) {
            const float v = a.dS_T ? a.dS_T[(((size_t)b * a.H + h) * D + 16 * vb + row) * D + col] : 0.f;
            sD[row * LS + col] = v;
            *p = v;
        } else {
            sD[row * LS + col] = *p;
        }
    }
    __syncthreads();

    auto step = [&](const O &o, int c) {
        // X = dS (D K)^T: value rows x tokens 16 w .. (A operand: dS rows r, k-contiguous)
        floatx4 acc = z4();
#pragma unroll
        for (int ks = 0; ks < O::KS; ++ks) {
            const floatx4 dv = *reinterpret_cast<const floatx4 *>(sD + r * LS + 16 * ks + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(dv[j], o.ka[ks][j], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sX[(4 * g + i) * LXX + 16 * w + r] = acc[i];
        gdn::lds_barrier();
        // the result: the previous chunk's exit-state gradient, or dS0 (the
        // sink if dS0 is not wanted); unconditional stores keep the wait counts exact
        float *dst = c > 0 ? record<D>(a, b, h, c - 1) + R::DSN
                           : (a.dS0 ? a.dS0 : a.sink) + ((size_t)b * a.H + h) * D * D;
#pragma unroll
        for (int j = 0; j < O::NTW; ++j) {
            const int nt = w + 4 * j;
            floatx4 d4, xw = z4(), oq = z4();
#pragma unroll
            for (int i = 0; i < 4; ++i) d4[i] = o.gC * sD[(4 * g + i) * LS + 16 * nt + r];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const floatx4 xv = *reinterpret_cast<const floatx4 *>(sX + r * LXX + 16 * ks + 4 * g);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    xw = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[jj], o.wb[j][ks][jj], xw, 0, 0, 0);
                    oq = __builtin_amdgcn_mfma_f32_16x16x4f32(o.oa[ks][jj], o.qb[j][ks][jj], oq, 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = d4[i] - xw[i] + oq[i];
                sD[(4 * g + i) * LS + 16 * nt + r] = v;
                dst[(16 * vb + 4 * g + i) * D + 16 * nt + r] = v;
            }
        }
        gdn::lds_barrier();
    };

    O oa, ob;
    rev_ops_load<D>(oa, recl, vb);
    for (int c = a.c1 - 1; c >= a.c0; c -= 2) {
        rev_ops_load<D>(ob, record<D>(a, b, h, max(c - 1, a.c0)), vb);
        __builtin_amdgcn_sched_barrier(0);
        step(oa, c);
        if (c - 1 < a.c0) break;
        rev_ops_load<D>(oa, record<D>(a, b, h, max(c - 2, a.c0)), vb);
        __builtin_amdgcn_sched_barrier(0);
        step(ob, c - 1);
    }
}

// ---------------------------------------------------------------------------
// Per chunk, given S (entry), dS' (exit-state gradient) and dO, wave w
// owning tokens 16w..16w+15 of every [64 x D] and [64 x 64] result:
//   U = U~ - W S^T
//   dU = P^T dO + diag(dl) K dS'^T          d dl = rowdot(K dS'^T, U)
//   dq^ = diag(gam) dO S + G K               d gam = rowdot(dO S, Q) + b rowdot(dR_W, K)
//   dk^ = diag(dl) U dS' + diag(b gam) dR_W + F K + F^T K + G^T Q
//   dW = -dU S,  dR_W = T^T dW,  dR_U = T^T dU,  dv^ = diag(b) dR_U
//   db = gam rowdot(dR_W, K) + rowdot(dR_U, V) + rowsum(dA o E o K K^T)
//   dA = -(dR_W W^T + dR_U U~^T) (strictly lower),  F = diag(b) (E o dA)
//   (E o K K^T, strictly lower, comes from the prep's record)
//   dP = dO U^T (lower-inclusive),  G = E o dP     (E_ij = e^{g_i - g_j})
//   dg = gam d gam - dl d dl + rowsum(M) - colsum(M),  M = dP o P + dA o A,
//        plus gC <dS', S> + sum(dl d dl) on the last token;
//   d log a = the suffix sums of dg inside the chunk.
template <int D>
__global__ __launch_bounds__(GNT) void bwd_grad_kernel(Args a) {
    typedef Rec<D> R;
    constexpr int LX = D + 4, LC = C + 4, NTH = D / 32;  // column tiles per wave
    extern __shared__ __align__(16) float lds[];
    float *L1 = lds, *L2 = L1 + C * LX, *L3 = L2 + C * LX;   // U then dR_W; dU; dW then dR_U
    float *La = L3 + C * LX, *Lb = La + C * LC, *Lc = Lb + C * LC;  // G; F; M
    float *vg = Lc + C * LC, *vb_ = vg + C, *vgam = vb_ + C, *vdl = vgam + C;
    float *vdgam = vdl + C, *vddl = vdgam + 2 * C, *vdb = vddl + 2 * C, *vred = vdb + 2 * C;
    const int c = a.c0 + blockIdx.x, h = blockIdx.y, b = blockIdx.z, t0 = c * C;
    // wave w: row block rb (tokens 16 rb ..), column tiles hf, hf + 2, hf + 4, ...
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, r = lane % 16, g = lane / 16;
    const int rb = w % 4, hf = w / 4;
    const float *rec = record<D>(a, b, h, c);
    const Seq sq = seq_of(a, b);

    if (tid < 64) {
        const int t = t0 + tid;
        const float gg = rec[R::G + tid];
        vg[tid] = gg;
        vb_[tid] = t < sq.len ? a.beta[((size_t)sq.off + src_t(a, sq, t)) * a.H + h] : 0.f;
        vgam[tid] = expf(gg);
        vdl[tid] = expf(rec[R::G + 63] - gg);
    }
    // <dS', S>
    {
        float s = 0.f;
        for (int idx = 4 * tid; idx < D * D; idx += 4 * GNT) {
            const floatx4 x = *reinterpret_cast<const floatx4 *>(rec + R::DSN + idx);
            const floatx4 y = *reinterpret_cast<const floatx4 *>(rec + R::SC + idx);
            s += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
        }
        s = wave_sum(s);
        if (lane == 0) vred[w] = s;
    }
    // U = U~ - W S^T
    {
        float af[D / 16][4];
        load_a<true, D>(af, rec + R::W, D, 16 * rb);
#pragma unroll 1
    for (int j = 0; j < NTH; ++j) {
        const int nt = 2 * j + hf;
        const floatx4 acc = mm16a<true, D>(z4(), af, rec + R::SC, D, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i, col = 16 * nt + r;
            L1[row * LX + col] = rec[R::UT + row * D + col] - acc[i];
        }
    }
    }
    __syncthreads();

    float pgam[4] = {0.f, 0.f, 0.f, 0.f}, pdl[4] = {0.f, 0.f, 0.f, 0.f}, pdb[4] = {0.f, 0.f, 0.f, 0.f};
    floatx4 dQ[NTH], dK[NTH];
    float rgam[4], rdl[4], rbb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * rb + 4 * g + i;
        rgam[i] = vgam[row];
        rdl[i] = vdl[row];
        rbb[i] = vb_[row];
    }
    // dU = P^T dO + diag(dl) K dS'^T, d dl
    {
        float ak[D / 16][4], ap[C / 16][4];
        load_a<true, D>(ak, rec + R::XK, D, 16 * rb);
        load_a<false, C>(ap, rec + R::P, C, 16 * rb);
#pragma unroll 1
    for (int j = 0; j < NTH; ++j) {
        const int nt = 2 * j + hf, col = 16 * nt + r;
        const floatx4 kd = mm16a<true, D>(z4(), ak, rec + R::DSN, D, 16 * nt);
        const floatx4 pt = mm16a<false, C>(z4(), ap, rec + R::DO, D, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i;
            L2[row * LX + col] = pt[i] + rdl[i] * kd[i];
            pdl[i] += kd[i] * L1[row * LX + col];
        }
    }
    }
    // dk^ = diag(dl) U dS'
#pragma unroll
    for (int j = 0; j < NTH; ++j) {
        const int nt = 2 * j + hf;
        const floatx4 uds = mm16<true, false, D>(z4(), L1, LX, 16 * rb, rec + R::DSN, D, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) dK[j][i] = rdl[i] * uds[i];
        __builtin_amdgcn_sched_barrier(0);
    }
    // dP = dO U^T (lower-inclusive): G = E o dP, M = dP o P; tiles hf, hf + 2
#pragma unroll 1
    for (int j = 0; j < 2; ++j) {
        const int nt = 2 * j + hf;
        floatx4 acc = z4();
        if (nt <= rb) acc = mm16<true, true, D>(acc, rec + R::DO, D, 16 * rb, L1, LX, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i, col = 16 * nt + r;
            const bool on = col <= row;
            La[row * LC + col] = on ? expf(vg[row] - vg[col]) * acc[i] : 0.f;
            Lc[row * LC + col] = on ? acc[i] * rec[R::P + row * C + col] : 0.f;
        }
    }
    __syncthreads();
    // dq^ = diag(gam) dO S, d gam, and dW = -dU S: each 16-key column block
    // of S is loaded once, for both products
    {
        float ad[D / 16][4];
        load_a<true, D>(ad, rec + R::DO, D, 16 * rb);
#pragma unroll
        for (int j = 0; j < NTH; ++j) {
            const int nt = 2 * j + hf, col = 16 * nt + r;
            float sb[D / 16][4];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sb[ks][jj] = rec[R::SC + (16 * ks + 4 * g + jj) * D + col];
            floatx4 dos = z4(), dw = z4();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const floatx4 u = *reinterpret_cast<const floatx4 *>(L2 + (16 * rb + r) * LX + 16 * ks + 4 * g);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    dos = __builtin_amdgcn_mfma_f32_16x16x4f32(ad[ks][jj], sb[ks][jj], dos, 0, 0, 0);
                    dw = __builtin_amdgcn_mfma_f32_16x16x4f32(u[jj], sb[ks][jj], dw, 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rb + 4 * g + i;
                dQ[j][i] = rgam[i] * dos[i];
                pgam[i] += dos[i] * rec[R::XQ + row * D + col];
                L3[row * LX + col] = -dw[i];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    // dR_W = T^T dW (into the U storage); T^T's rows are held for dR_U too
    float at[C / 16][4];
    load_a<false, C>(at, rec + R::TM, C, 16 * rb);
#pragma unroll
    for (int j = 0; j < NTH; ++j) {
        const int nt = 2 * j + hf, col = 16 * nt + r;
        const floatx4 acc = mm16a<false, C>(z4(), at, L3, LX, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i;
            L1[row * LX + col] = acc[i];
            dK[j][i] += rbb[i] * rgam[i] * acc[i];
            const float rk = acc[i] * rec[R::XK + row * D + col];
            pgam[i] += rbb[i] * rk;
            pdb[i] += rgam[i] * rk;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // dR_U = T^T dU (into the dW storage), dv^ = diag(b) dR_U
    float *dxv = const_cast<float *>(rec) + R::DXV;
#pragma unroll 1
    for (int j = 0; j < NTH; ++j) {
        const int nt = 2 * j + hf, col = 16 * nt + r;
        const floatx4 acc = mm16a<false, C>(z4(), at, L2, LX, 16 * nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i;
            L3[row * LX + col] = acc[i];
            dxv[row * D + col] = rbb[i] * acc[i];
            pdb[i] += acc[i] * rec[R::XV + row * D + col];
        }
    }
    __syncthreads();
    // dA = -(dR_W W^T + dR_U U~^T) (strictly lower), F = diag(b) (E o dA), M += dA o A
#pragma unroll 1
    for (int j = 0; j < 2; ++j) {
        const int nt = 2 * j + hf;
        floatx4 acc = z4();
        if (nt <= rb) {
            acc = mm16<true, true, D>(acc, L1, LX, 16 * rb, rec + R::W, D, 16 * nt);
            acc = mm16<true, true, D>(acc, L3, LX, 16 * rb, rec + R::UT, D, 16 * nt);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i, col = 16 * nt + r;
            float f = 0.f;
            if (col < row) {
                // E o K K^T from the prep (so A = diag(b) of it)
                const float e = expf(vg[row] - vg[col]), da = -acc[i], ekk = rec[R::EKK + row * C + col];
                f = rbb[i] * e * da;
                pdb[i] += da * ekk;
                Lc[row * LC + col] += rbb[i] * da * ekk;
            }
            Lb[row * LC + col] = f;
        }
    }
    __syncthreads();
    // dk^ += F K + F^T K + G^T Q;  dq^ += G K.  The A operands (rows and
    // columns 16 rb .. of F and G) are held for all column tiles, and each
    // column block of K serves three products.
    float *dxq = const_cast<float *>(rec) + R::DXQ, *dxk = const_cast<float *>(rec) + R::DXK;
    float fa[C / 16][4], fta[C / 16][4], ga[C / 16][4], gta[C / 16][4];
    load_a<true, C>(fa, Lb, LC, 16 * rb);
    load_a<false, C>(fta, Lb, LC, 16 * rb);
    load_a<true, C>(ga, La, LC, 16 * rb);
    load_a<false, C>(gta, La, LC, 16 * rb);
#pragma unroll
    for (int j = 0; j < NTH; ++j) {
        const int nt = 2 * j + hf;
        float kb[C / 16][4], qb[C / 16][4];
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                kb[ks][jj] = rec[R::XK + (16 * ks + 4 * g + jj) * D + 16 * nt + r];
                qb[ks][jj] = rec[R::XQ + (16 * ks + 4 * g + jj) * D + 16 * nt + r];
            }
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                dK[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[ks][jj], kb[ks][jj], dK[j], 0, 0, 0);
                dK[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fta[ks][jj], kb[ks][jj], dK[j], 0, 0, 0);
                dK[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(gta[ks][jj], qb[ks][jj], dK[j], 0, 0, 0);
                dQ[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[ks][jj], kb[ks][jj], dQ[j], 0, 0, 0);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * g + i, col = 16 * nt + r;
            dxq[row * D + col] = dQ[j][i];
            dxk[row * D + col] = dK[j][i];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // per-row sums over the 16 lanes of a row, one set per column half
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float sg_ = gdn::group_sum<16>(pgam[i]), sd = gdn::group_sum<16>(pdl[i]), sb = gdn::group_sum<16>(pdb[i]);
        if (r == 0) {
            const int row = 16 * rb + 4 * g + i;
            vdgam[hf * C + row] = sg_;
            vddl[hf * C + row] = sd;
            vdb[hf * C + row] = sb;
        }
    }
    __syncthreads();
    if (tid < 64) {
        const int t = tid;
        float rs = 0.f, cs = 0.f;
        for (int j = 0; j < 64; ++j) {
            rs += Lc[t * LC + j];
            cs += Lc[j * LC + t];
        }
        const float ddl = vddl[t] + vddl[C + t], dgam = vdgam[t] + vdgam[C + t];
        const float e = vdl[t] * ddl;
        float dg = vgam[t] * dgam - e + rs - cs;
        const float tot = wave_sum(e);
        float red = 0.f;
#pragma unroll
        for (int q = 0; q < GW; ++q) red += vred[q];
        if (t == 63) dg += rec[R::G + 64] * red + tot;
        // suffix sums: d log a_t = sum over r >= t of dg_r
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_down(dg, o, 64);
            if (t + o < 64) dg += y;
        }
        const int tt = t0 + t;
        if (tt < sq.len) {
            const size_t row = (size_t)sq.off + src_t(a, sq, tt);
            a.dlog_a[row * a.H + h] = dg;
            a.dbeta[row * a.H + h] = vdb[t] + vdb[C + t];
        }
    }
}

// ---------------------------------------------------------------------------
// Per chunk, for q, k and v in turn: the backward of the L2 norm (q, k) and
// of SiLU for the chunk's 64 tokens and the next 3 (dz, kept in LDS), then
// dx_t = sum_j w_j dz_{t+3-j} (dz zero past the end) and the chunk's sums
// dz_t x_{t-3+j} for the conv weights.  Thread: 8 channels of RUN
// consecutive rows; its raw rows (RUN + 3, with the conv history) are loaded
// once and serve the conv, its recomputation and the weight sums.
template <int D> struct PrologueCfg {
    static constexpr int G = D / 8, RUNS = NT / G, RUN = (C + 3 + RUNS - 1) / RUNS, ROWS = RUN + 3;
    static constexpr int LZ = D + 4;
};

template <class IO, int D>
__global__ __launch_bounds__(NT) void bwd_prologue_kernel(Args a) {
    typedef Rec<D> R;
    typedef PrologueCfg<D> P;
    constexpr int G = P::G, RUN = P::RUN, ROWS = P::ROWS, LZ = P::LZ;
    extern __shared__ __align__(16) float lds[];
    float *sZ = lds;                    // dz, rows 0..66 of the chunk
    float *sW = sZ + (C + 3) * LZ;      // conv-weight partial sums [RUNS][D * 4]
    const int c = a.c0 + blockIdx.x, h = blockIdx.y, b = blockIdx.z, t0 = c * C;
    const int tid = threadIdx.x, cg = tid % G, run = tid / G, r0 = run * RUN;
    const Seq sq = seq_of(a, b);
    const IO *src[3] = {static_cast<const IO *>(a.q), static_cast<const IO *>(a.k), static_cast<const IO *>(a.v)};
    IO *dst[3] = {static_cast<IO *>(a.dq), static_cast<IO *>(a.dk), static_cast<IO *>(a.dv)};
    const float *cw[3] = {a.conv_q, a.conv_k, a.conv_v};
    const int dxo[3] = {R::DXQ, R::DXK, R::DXV};
#pragma unroll 1
    for (int x = 0; x < 3; ++x) {
        Row8<IO> raw[ROWS];
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr) {
            const int sp = t0 + r0 - 3 + rr;
            const bool ok = sp >= 0 && sp < sq.len;
            raw[rr].load(src[x] + ((((size_t)sq.off + (ok ? src_t(a, sq, sp) : 0)) * a.H + h) * D) + 8 * cg, ok);
        }
        floatx4 dxh[RUN][2];
#pragma unroll
        for (int rt = 0; rt < RUN; ++rt) {
            const int t = t0 + r0 + rt;
            const bool ok = t < sq.len && r0 + rt < C + 3;
            const float *pr = ok ? record<D>(a, b, h, t / C) + dxo[x] + (t % C) * D + 8 * cg : nullptr;
            dxh[rt][0] = ok ? *reinterpret_cast<const floatx4 *>(pr) : z4();
            dxh[rt][1] = ok ? *reinterpret_cast<const floatx4 *>(pr + 4) : z4();
        }
        float wt[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 wv = *reinterpret_cast<const float4 *>(cw[x] + ((size_t)h * D + 8 * cg + i) * 4);
            wt[i][0] = wv.x; wt[i][1] = wv.y; wt[i][2] = wv.z; wt[i][3] = wv.w;
        }
        float pw[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) pw[i][j] = 0.f;
#pragma unroll
        for (int rt = 0; rt < RUN; ++rt) {
            const int tl = r0 + rt, t = t0 + tl;
            float z[8], sv[8], dv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float zz = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) zz = fmaf(wt[i][j], raw[rt + j].get(i), zz);
                z[i] = zz;
                sv[i] = silu(zz);
                dv[i] = dxh[rt][i / 4][i % 4];
            }
            if (x < 2) {
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) ss += sv[i] * sv[i];
                ss = gdn::group_sum<G>(ss);
                const float rho = 1.0f / sqrtf(ss + a.eps_l2);
                float dot = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) dot += sv[i] * rho * dv[i];
                dot = gdn::group_sum<G>(dot);
#pragma unroll
                for (int i = 0; i < 8; ++i) dv[i] = rho * (dv[i] - sv[i] * rho * dot);
            }
            const bool valid = t < sq.len;
            float dz[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) dz[i] = valid ? dv[i] * dsilu(z[i]) : 0.f;
            if (tl < C + 3) {
                float *row = sZ + tl * LZ + 8 * cg;
                *reinterpret_cast<float4 *>(row) = make_float4(dz[0], dz[1], dz[2], dz[3]);
                *reinterpret_cast<float4 *>(row + 4) = make_float4(dz[4], dz[5], dz[6], dz[7]);
            }
            if (tl < C) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) pw[i][j] = fmaf(dz[i], raw[rt + j].get(i), pw[i][j]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<float4 *>(sW + run * (D * 4) + (8 * cg + i) * 4) =
                make_float4(pw[i][0], pw[i][1], pw[i][2], pw[i][3]);
        __syncthreads();
        // dx for the chunk's tokens
#pragma unroll
        for (int rt = 0; rt < RUN; ++rt) {
            const int tl = r0 + rt, t = t0 + tl;
            if (tl < C && t < sq.len) {
                float dx[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc = fmaf(wt[i][j], sZ[(tl + 3 - j) * LZ + 8 * cg + i], acc);
                    dx[i] = acc;
                }
                IO *o = dst[x] + (((size_t)sq.off + src_t(a, sq, t)) * a.H + h) * D + 8 * cg;
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = (IO)dx[i];
            }
        }
        // the chunk's conv-weight sums, over the runs in a fixed order
        for (int e = tid; e < D * 4; e += NT) {
            float sum = 0.f;
            for (int q = 0; q < P::RUNS; ++q) sum += sW[q * (D * 4) + e];
            a.part_conv[(((size_t)b * a.NC + c) * a.H + h) * (3 * D * 4) + x * D * 4 + e] = sum;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// The conv weights' and the norm weight's gradients: sums of the per-chunk
// parts over batch rows and chunks, in a fixed order.
template <int D>
__global__ __launch_bounds__(NT) void bwd_reduce_kernel(Args a) {
    // 64 outputs per workgroup; wave s sums slice s of the (batch row,
    // chunk) parts, and the 4 slice sums are added in order
    constexpr int SL = NT / 64;
    __shared__ float sp[SL][64];
    const int e = blockIdx.x * 64 + threadIdx.x % 64, sl = threadIdx.x / 64;
    const int nconv = a.H * 3 * D * 4, ntot = nconv + a.H * D;
    const int nbc = a.B * a.NC, per = (nbc + SL - 1) / SL, b0 = sl * per, b1 = min(nbc, b0 + per);
    float s = 0.f;
    if (e < nconv) {
        const int h = e / (3 * D * 4), rem = e % (3 * D * 4);
#pragma unroll 8
        for (int bc = b0; bc < b1; ++bc) s += a.part_conv[((size_t)bc * a.H + h) * (3 * D * 4) + rem];
    } else if (e < ntot) {
        const int j = e - nconv, h = j / D, ch = j % D;
#pragma unroll 8
        for (int bc = b0; bc < b1; ++bc) s += a.part_norm[((size_t)bc * a.H + h) * D + ch];
    }
    sp[sl][threadIdx.x % 64] = s;
    __syncthreads();
    if (sl == 0 && e < ntot) {
        float t = sp[0][threadIdx.x];
#pragma unroll
        for (int q = 1; q < SL; ++q) t += sp[q][threadIdx.x];
        if (e < nconv) {
            const int h = e / (3 * D * 4), rem = e % (3 * D * 4), x = rem / (D * 4), f = rem % (D * 4);
            float *dst = x == 0 ? a.dconv_q : (x == 1 ? a.dconv_k : a.dconv_v);
            dst[(size_t)h * D * 4 + f] = t;
        } else if (a.dnorm_w) {
            a.dnorm_w[e - nconv] = t;
        }
    }
}

}  // namespace gdnb

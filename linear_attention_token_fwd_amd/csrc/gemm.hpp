// gemm.hpp -- the token mixer's projections on gfx950 bf16 MFMA.
//
// The GDN module takes its per-token inputs from the hidden states through
// linear projections and hands its output back through one (LinMorph project
// page, "Why learn the initialization?": the GDN parameters are built from
// the pretrained query, key, value and output projections; the QKV and O
// projections are the "QKV proj." and "O proj." columns of the T3-Video
// page's Table 1).  Both are products  out[M, N] = X[M, K] W[N, K]^T (+ bias)
// with K-contiguous rows on both sides, the layout of a linear layer's
// weight.  The in-projection's epilogue also does the gate
// parameterisation:  b = sigmoid(z_b),  log a = -exp(A_h) softplus(z_a).
//
// Tiling.  One workgroup of 8 waves (two per SIMD, so one wave's LDS reads
// hide behind the other's MFMAs) computes a 256 x 256 output tile over K in
// steps of 64.  The operand tiles of a step (256 rows of X and 256 rows of
// W, 128 bytes each, 64 KB) are copied global -> LDS by direct-to-LDS loads
// (16 B per lane, 8 rows x 128 B per load, so each row is one whole cache
// line) into a ring of 2 stages: the copy of step s + 1 runs while step s is
// multiplied.  In LDS the 16-byte chunks of a row are XOR-swizzled by the row
// so that the fragment reads are free of bank conflicts.  Wave (wm, wn) owns
// the 128 x 64 sub-tile (8 x 4 MFMA tiles of 16 x 16) and reads each W
// fragment from LDS while the MFMAs of the previous one run.  (Four waves
// with 128 x 128 sub-tiles: 853 against 1023 TFLOP/s for the in-projection
// at M = 32760, N = 6168, K = 1536.)
//
// Operand order.  The MFMA's A operand is W and its B operand is X, so the
// accumulator tile is out^T: lane (r, g) holds out[m + r][n + 4g .. 4g+3],
// four consecutive columns of one row, stored as one 8-byte write.
#pragma once
#include "frag.hpp"
#include "sync.hpp"

namespace gdn {

namespace gemm {
constexpr int BM = 256;        // output rows (X rows) per workgroup
constexpr int BN = 256;        // output columns (W rows) per workgroup
constexpr int BK = 64;         // k per step (one 128-byte line of each row)
constexpr int STAGES = 2;      // LDS ring depth
constexpr int UNIT = 1024;     // bytes of one copy unit: 8 rows x 128 B
constexpr int XU = BM / 8;     // X units per step
constexpr int WU = BN / 8;     // W units per step
constexpr int STAGE_BYTES = (XU + WU) * UNIT;     // 64 KB
constexpr int EPI_LD = 144;     // bytes per staged output row (64 bf16 + 16 B pad)
constexpr int EPI_WAVE = 128 * EPI_LD;            // one wave's 128 x 64 output block
constexpr int LDS_BYTES = STAGES * STAGE_BYTES > 8 * EPI_WAVE ? STAGES * STAGE_BYTES : 8 * EPI_WAVE;  // 144 KB
constexpr int THREADS = 512;
constexpr int DMA_PER_WAVE = (XU + WU) / (THREADS / 64);  // 8
constexpr int GROUP_M = 4;     // row tiles per group of the tile order
}  // namespace gemm

enum GemmEpilogue { kEpiPlain = 0, kEpiInProj = 1 };

struct GemmArgs {
    int M, N, K;
    int mt, nt;                // tiles along M and N
    const bf16 *x;             // [M, K]
    const bf16 *w;             // [N, K]
    const float *bias;         // [N] or null
    // plain epilogue: out[M, N]
    bf16 *out;
    // in-projection epilogue: columns [0, 4HD) go to q, k, v, gate ([M, HD]
    // each); column 4HD + j to b (j < H) or log a (H <= j < 2H), [M, H] each
    bf16 *dst[4];
    int HD, H;
    float *beta, *log_a;
    const float *A_log;        // [H]
};

// Position of workgroup L in the tile order: tiles in groups of GROUP_M row
// tiles, column-major inside a group, so the workgroups running together on
// one XCD share X rows and W rows in its L2.
__device__ __forceinline__ bool gemm_tile(const GemmArgs &a, int &tm, int &tn) {
    int p;
    if (!xcd_position(blockIdx.x, a.mt * a.nt, gridDim.x, p)) return false;
    const int per_group = gemm::GROUP_M * a.nt;
    const int grp = p / per_group, in = p % per_group;
    const int gm = min(gemm::GROUP_M, a.mt - grp * gemm::GROUP_M);
    tn = in / gm;
    tm = grp * gemm::GROUP_M + in % gm;
    return true;
}

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float softplus_f(float z) { return z > 20.0f ? z : log1pf(expf(z)); }

__device__ __forceinline__ floatx4 add_bias4(const float *bias, int col, floatx4 v) {
    if (bias) {
        const float4 bv = *reinterpret_cast<const float4 *>(bias + col);
        v[0] += bv.x; v[1] += bv.y; v[2] += bv.z; v[3] += bv.w;
    }
    return v;
}

__device__ __forceinline__ void store_bf16x4(bf16 *p, floatx4 v) {
    bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *reinterpret_cast<bf16x4 *>(p) = o;
}

template <int EPI>
__global__ __launch_bounds__(gemm::THREADS, 2) void gdn_gemm_kernel(GemmArgs a) {
    using namespace gemm;
    typedef Mfma<bf16> Mf;
    typedef Mf::frag frag;
    extern __shared__ __align__(16) unsigned char smem[];

    int tm, tn;
    if (!gemm_tile(a, tm, tn)) return;
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid % 64, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm = w & 1, wn = w >> 1;

    // Copies.  A step holds, for each of the 512 rows (256 of X, then 256 of
    // W), the 128 bytes k = 64 s .. 64 s + 63 of that row, as 64 units of 8
    // rows x 128 B; one direct-to-LDS load (16 B per lane) fills one unit, so
    // every row is read as one whole 128-byte line.  Lane L of a unit loads
    // 16-byte chunk c = (L % 8) ^ (L / 8) of row L / 8: chunk c of row r' sits
    // in slot 8 r' + (c ^ r').  A 128-bit LDS read is served 8 lanes at a
    // time, and the swizzle puts the 8 rows such a group reads (the same
    // chunk of rows r' = 0..7) on 8 distinct 16-byte bank groups.
    // Waves 0-3 copy the X units, waves 4-7 the W units.  Rows past the end
    // read the last row (never stored).  Element offsets fit in 32 bits (the
    // host checks M K and N K).
    const bf16 *base = w < 4 ? a.x : a.w;
    unsigned off[DMA_PER_WAVE];
    {
        const int rr = lane >> 3, chunk = (lane & 7) ^ rr;
#pragma unroll
        for (int b = 0; b < DMA_PER_WAVE; ++b) {
            const int u = w * DMA_PER_WAVE + b;  // unit of the step
            const int row = u < XU ? min(m0 + 8 * u + rr, a.M - 1) : min(n0 + 8 * (u - XU) + rr, a.N - 1);
            off[b] = (unsigned)row * (unsigned)a.K + 8 * chunk;
        }
    }
    auto issue = [&](int s) {
        unsigned char *dst = smem + (s % STAGES) * STAGE_BYTES + w * DMA_PER_WAVE * UNIT;
#pragma unroll
        for (int b = 0; b < DMA_PER_WAVE; ++b)
            __builtin_amdgcn_global_load_lds(base + off[b] + s * BK, dst + b * UNIT, 16, 0, 0);
    };
    // Fragment reads.  Lane (r, g) of a 16-row fragment tile t (units 2t and
    // 2t + 1) reads row r, chunk c = 4 kb + g of k-block kb.
    unsigned fo[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int rr = r & 7, hi = r >> 3;
        fo[kb] = hi * UNIT + (8 * rr + ((4 * kb + g) ^ rr)) * 16;
    }

    floatx4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = zero4();

    // Pipeline: the copy of step s + 1 runs while step s is multiplied.
    // Iteration s: wait for this wave's copies of step s and barrier (every
    // wave's copies have landed, and every wave is done reading step s - 1,
    // whose stage the copy of step s + 1 reuses); issue that copy; multiply
    // step s, reading each W fragment while the MFMAs of the previous one run.
    const int S = a.K / BK;
    issue(0);
    // A step is 8 groups (kb, i) of 8 MFMAs sharing W fragment (kb, i) and
    // the 8 X fragments of kb.  W fragments are read two groups ahead, the X
    // fragments of kb = 1 during kb = 0.
    frag xf[2][8], wf[3];
    // 16-column tiles of this wave that hold output columns (fewer only in
    // the last column tile: N = 4 H D + 2 H leaves its gate columns there)
    const int live_tiles = min(4, max(0, (a.N - (n0 + 64 * wn) + 15) / 16));
    for (int s = 0; s < S; ++s) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();
        if (s + 1 < S) issue(s + 1);
        const unsigned char *buf = smem + (s % STAGES) * STAGE_BYTES;
        auto wfrag = [&](int q) {  // W fragment of group q = 4 kb + i
            return *reinterpret_cast<const frag *>(buf + 2 * (XU / 2 + 4 * wn + (q & 3)) * UNIT + fo[q >> 2]);
        };
        auto xfrag = [&](int kb, int j) {
            return *reinterpret_cast<const frag *>(buf + 2 * (8 * wm + j) * UNIT + fo[kb]);
        };
#pragma unroll
        for (int j = 0; j < 8; ++j) xf[0][j] = xfrag(0, j);
        wf[0] = wfrag(0);
        wf[1] = wfrag(1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q + 2 < 8) wf[(q + 2) % 3] = wfrag(q + 2);
            if (q < 4) {
                xf[1][2 * q] = xfrag(1, 2 * q);
                xf[1][2 * q + 1] = xfrag(1, 2 * q + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            if ((q & 3) < live_tiles) {
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[q & 3][j] = Mf::mma(wf[q % 3], xf[q >> 2][j], acc[q & 3][j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Epilogue.  acc[i][j]: lane (r, g) holds out[m0 + 128 wm + 16 j + r][n0 +
    // 64 wn + 16 i + 4g .. +3].  The in-projection's gate columns (past
    // 4 H D) go out from registers, element by element; every other value,
    // bias added, is staged as bf16 in LDS (each wave its own 128 x 64 block,
    // rows padded to 144 B) and stored from there as 16-byte pieces of whole
    // 128-byte row segments.
    const int row0 = m0 + 128 * wm, col0 = n0 + 64 * wn;
    const int ncols = EPI == kEpiPlain ? a.N : min(a.N, 4 * a.HD);  // columns staged and stored from LDS
    if (EPI == kEpiInProj) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tcol = col0 + 16 * i;  // wave-uniform
            if (tcol + 16 <= 4 * a.HD || tcol >= a.N) continue;
            const int col = tcol + 4 * g;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = row0 + 16 * j + r;
                if (row >= a.M) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jj = col + e - 4 * a.HD;
                    if (jj < 0 || jj >= 2 * a.H) continue;
                    const float z = acc[i][j][e] + (a.bias ? a.bias[col + e] : 0.f);
                    if (jj < a.H)
                        a.beta[(size_t)row * a.H + jj] = sigmoid_f(z);
                    else
                        a.log_a[(size_t)row * a.H + (jj - a.H)] = -expf(a.A_log[jj - a.H]) * softplus_f(z);
                }
            }
        }
    }
    lds_barrier();  // every wave is done with the operand stages
    unsigned char *stage = smem + w * EPI_WAVE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = col0 + 16 * i + 4 * g;
        const floatx4 bv = col + 4 <= ncols ? add_bias4(a.bias, col, zero4()) : zero4();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const floatx4 v = acc[i][j] + bv;
            bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
            *reinterpret_cast<bf16x4 *>(stage + (16 * j + r) * EPI_LD + (16 * i + 4 * g) * 2) = o;
        }
    }
    __builtin_amdgcn_s_waitcnt(kLgkm0);  // this wave's block is in LDS (only this wave reads it)
    // 8 lanes per row, 8 columns (16 B) each, 8 rows per pass
    const int lr = lane / 8, lc = 8 * (lane % 8);
    const int col = col0 + lc;
    if (col < ncols) {
        bf16 *dst;
        size_t ld;
        if (EPI == kEpiPlain) {
            dst = a.out + col;
            ld = a.N;
        } else {
            const int part = col / a.HD;
            bf16 *base = part == 0 ? a.dst[0] : part == 1 ? a.dst[1] : part == 2 ? a.dst[2] : a.dst[3];
            dst = base + (col - part * a.HD);
            ld = a.HD;
        }
        const bool full = col + 8 <= ncols;  // else 4 columns (ncols % 4 == 0)
#pragma unroll 4
        for (int pass = 0; pass < 16; ++pass) {
            const int rr = 8 * pass + lr;
            const int row = row0 + rr;
            if (row >= a.M) break;
            const unsigned char *src = stage + rr * EPI_LD + lc * 2;
            if (full)
                *reinterpret_cast<bf16x8 *>(dst + (size_t)row * ld) = *reinterpret_cast<const bf16x8 *>(src);
            else
                *reinterpret_cast<bf16x4 *>(dst + (size_t)row * ld) = *reinterpret_cast<const bf16x4 *>(src);
        }
    }
}

}  // namespace gdn

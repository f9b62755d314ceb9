// frag.hpp -- CDNA4 (gfx950) MFMA tiles used by the GDN kernels.
//
// All products use 16x16 output tiles on a 64-lane wave:
//   bf16 operands: v_mfma_f32_16x16x32_bf16  (8 bf16 per lane per operand)
//   fp32 operands: v_mfma_f32_16x16x4_f32    (1 fp32 per lane per operand)
// Lane l = 16*g + r (g = l/16 "lane group", r = l%16).
//   A operand (16 x K):  lane (r, g) holds row r.
//   B operand (K x 16):  lane (r, g) holds column r.
//   C/D tile  (16 x 16): lane (r, g) holds rows 4g+i (i = 0..3) of column r.
//
// K order.  The hardware pairs the A and B values that sit in the same lane
// group and slot, so any bijection between (group, slot) and k gives the same
// product as long as A and B use the same one.  Every operand here uses the
// "tile-chained" order, in which a lane's flat element e (over a K range that
// is a multiple of 16) stands for
//        k(e, g) = 16 * (e / 4) + 4 * g + (e % 4)
// and fragment kb holds elements e = kb*KPL .. kb*KPL + KPL-1.  In this order
// the 4 values a lane holds of a C tile covering rows 16m..16m+15 are exactly
// its elements e = 4m..4m+3, so a product's output tiles feed the next
// product as its B operand without leaving the lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kWaves = 4;   // waves per workgroup
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ int kchain(int e, int g) { return 16 * (e >> 2) + 4 * g + (e & 3); }

template <class OT> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int KPL = 8;  // k values per lane per operand
    static constexpr int K = 32;   // k per instruction
    typedef bf16x8 frag;
    static __device__ __forceinline__ floatx4 mma(const frag &a, const frag &b, const floatx4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    static constexpr int KPL = 1;
    static constexpr int K = 4;
    typedef float frag;
    static __device__ __forceinline__ floatx4 mma(const frag &a, const frag &b, const floatx4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// element access on a fragment (bf16x8 or float)
__device__ __forceinline__ void fset(bf16x8 &f, int j, float x) { f[j] = (bf16)x; }
__device__ __forceinline__ void fset(float &f, int, float x) { f = x; }
__device__ __forceinline__ float fget(const bf16x8 &f, int j) { return (float)f[j]; }
__device__ __forceinline__ float fget(const float &f, int) { return f; }

template <class OT> __device__ __forceinline__ OT to_ot(float x) { return (OT)x; }

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

// SiLU with the hardware reciprocal (about 1 ulp) in place of an IEEE divide:
// z / (1 + e^-z) is z * rcp(1 + e^-z); for large -z, e^-z = inf gives -0.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
// 1 / sqrt(x) with the hardware reciprocal square root (about 1 ulp)
__device__ __forceinline__ float rsqrt_fast(float x) { return __builtin_amdgcn_rsqf(x); }

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// Sum over aligned groups of N = 8 or 16 consecutive lanes, every lane of a
// group receiving the group's sum, by DPP lane permutations (no LDS): swap
// neighbours, swap pairs (quad_perm), then mirror each half row (lanes 0-3
// <-> 7-4 of every 8) and, for 16, each row (lanes 0-7 <-> 15-8).  After the
// quad steps the four lanes of a quad hold the same value, so a mirror adds
// the other quad's (or half row's) total.
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int N> __device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    x += dpp_f<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp_f<0x141>(x);  // row_half_mirror
    if constexpr (N == 16) x += dpp_f<0x140>(x);  // row_mirror
    return x;
}

}  // namespace gdn

// sync.hpp -- barriers, wait counts and XCD-aware workgroup placement for
// the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

// Barriers that do not wait for vector memory.  The compiler fences and
// scheduling barriers keep it from moving memory accesses (or any other
// instruction) across the barrier; lds_barrier() also waits for this wave's
// LDS accesses so that its LDS writes are visible after it.
__device__ __forceinline__ void bare_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// s_waitcnt immediate for "at most n vector memory operations outstanding"
// (gfx9 encoding; the LDS and export counters are left unconstrained).
constexpr unsigned vmcnt_imm(unsigned n) { return (n & 0xFu) | ((n >> 4) << 14) | (0x7u << 4) | (0xFu << 8); }
constexpr unsigned kLgkm0 = 0xF | (0x3u << 14) | (0x7u << 4);  // lgkmcnt(0), others unconstrained
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    bare_barrier();
}

// Workgroup placement: launched as a 1-D grid whose size is a multiple of 8.
// Consecutive workgroup ids go to different XCDs (round robin), so id L is
// mapped to position p = (L % 8) * per + L / 8 of the kernel's ordered work
// list: each XCD gets one contiguous eighth of the list, and neighbours in
// the list share that XCD's L2.
__device__ __forceinline__ bool xcd_position(int L, int nwg_used, int nwg_launched, int &p) {
    const int per = nwg_launched / 8;
    p = (L % 8) * per + L / 8;
    return p < nwg_used;
}

}  // namespace gdn

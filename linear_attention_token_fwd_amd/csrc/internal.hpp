// internal.hpp -- functions shared between the library's translation units
// (hidden: not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/gdn.h"

namespace gdn_internal {

#define GDN_HIDDEN __attribute__((visibility("hidden")))

// The I/O dtype as the int a C caller stored.  A C struct may hold any int in
// an enum field, but in C++ loading an enum object whose value lies outside
// the enumeration's range is undefined behaviour, so the checks read the
// field's bytes as an int; once a value has passed them, the field is read
// as the enum.
// base + off bytes, computed on the address's integer value: the plan
// builders also run for sizes only (launch counts and names), with a NULL
// workspace, where pointer arithmetic would be undefined.
template <class T = char> inline T *at_offset(const void *base, size_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<uintptr_t>(base) + off);
}

inline int dtype_code(const gdn_dtype &d) {
    static_assert(sizeof(gdn_dtype) == sizeof(int), "gdn_dtype is stored as an int");
    int v;
    __builtin_memcpy(&v, &d, sizeof v);
    return v;
}

// A kernel launch of another part of the library, placed inside a layer
// call's launch plan (the argument bytes are copied).
struct ExtLaunch {
    const void *fn;
    dim3 grid, block;
    size_t smem;
    unsigned char args[160];
    const char *name;
};

// Every check gdn_fwd makes, without launching anything.
GDN_HIDDEN gdn_status fwd_check(const gdn_fwd_params *p);
// The chunk ranges a one-scan layer call runs: R + 1 bounds in chunks, 0 first
// and ceil(T / 64) last; range i is chunks [bounds[i], bounds[i+1]) of every
// batch row.
GDN_HIDDEN void scan_range_bounds(const gdn_fwd_params *p, std::vector<int> &bounds);
// gdn_fwd (one scan, equal lengths) with other launches woven into its plan:
// post[i] (one entry per range) runs after the output kernel of range i, on
// a library stream, in range order.  Nothing is checked here beyond what
// gdn_fwd checks.
GDN_HIDDEN gdn_status fwd_call_staged(const gdn_fwd_params *p, const std::vector<std::vector<ExtLaunch>> &post,
                                      hipStream_t s);
// gdn_fwd / gdn_fwd_timed (timing: NULL, or 2 events per launch).
GDN_HIDDEN gdn_status fwd_call(const gdn_fwd_params *p, hipEvent_t *timing, int n_timing, hipStream_t s);

}  // namespace gdn_internal

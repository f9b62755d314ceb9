// internal.hpp -- functions shared between the library's translation units
// (hidden: not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/gdn.h"

namespace gdn_internal {

#define GDN_HIDDEN __attribute__((visibility("hidden")))

// Every check gdn_fwd makes, without launching anything.
GDN_HIDDEN gdn_status fwd_check(const gdn_fwd_params *p);
// gdn_fwd / gdn_fwd_timed (timing: NULL, or 2 events per launch).
GDN_HIDDEN gdn_status fwd_call(const gdn_fwd_params *p, hipEvent_t *timing, int n_timing, hipStream_t s);

}  // namespace gdn_internal

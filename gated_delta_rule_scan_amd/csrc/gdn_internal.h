// Internal launch entry points of the libgdn kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_common.h"

namespace gdn {

// State-independent chunk quantities (triangular inverses, decayed q.k,
// per-token scales); zeroes the output rows of its chunk when a.zero_out is
// set (bidirectional scans accumulate into it).  Grid: (NC, B*H).
template <typename MT, int DK, int C>
hipError_t launch_prep(const ScanArgs& a, hipStream_t stream);

// Sequential inter-chunk state chain with the chunk outputs fused in.
// NT: 16-column value tiles per workgroup; ACC: bidirectional (one workgroup
// per direction, readouts added into the output that the preparation kernel
// zeroed) instead of one direction (`rev_single` tells which) stored directly.
template <typename MT, int DK, int C, int NT, bool ACC>
hipError_t launch_chain(const ScanArgs& a, int rev_single, hipStream_t stream);

}  // namespace gdn

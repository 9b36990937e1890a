// Internal launch entry points of the libgdn kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_common.h"

namespace gdn {

// State-independent chunk quantities (triangular inverses, decayed q.k,
// per-token scales).  Grid: (NC, B*H).
template <typename MT, int DK, int C>
hipError_t launch_prep(const ScanArgs& a, hipStream_t stream);

// Sequential inter-chunk state chain with the chunk outputs fused in.
// NT: 16-column value tiles per workgroup; DIRS: direction groups per
// workgroup (2 = forward and reverse of the same tile together).
template <typename MT, int DK, int C, int NT, int DIRS>
hipError_t launch_chain(const ScanArgs& a, int rev_single, hipStream_t stream);

}  // namespace gdn

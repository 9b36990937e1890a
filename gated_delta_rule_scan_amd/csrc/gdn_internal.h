// Internal launch entry points of the libgdn kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_common.h"

namespace gdn {

// State-independent chunk quantities (triangular inverses, decayed q.k,
// per-token scales); fills the output rows of its chunk with the "not written
// yet" pattern when a.zero_out is set (bidirectional scans).  Grid: (NC, B*H).
template <typename MT, int DK, int C>
hipError_t launch_prep(const ScanArgs& a, hipStream_t stream);

// Sequential inter-chunk state chain with the chunk outputs fused in.
// NT: 16-column value tiles per workgroup; BI: bidirectional (one workgroup
// per direction; the second visitor of a chunk adds the first one's readout,
// which it recognises against the pattern the preparation kernel filled the
// output with) instead of one direction (`rev_single` tells which).
template <typename MT, int DK, int C, int NT, bool BI>
hipError_t launch_chain(const ScanArgs& a, int rev_single, hipStream_t stream);

}  // namespace gdn

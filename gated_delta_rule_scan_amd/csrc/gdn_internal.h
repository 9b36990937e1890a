// Internal launch entry points of the libgdn kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_common.h"

namespace gdn {

// State-independent chunk quantities (triangular inverses, decayed q.k,
// per-token scales); fills the output rows of its chunk with the "not written
// yet" pattern when a.zero_out is set (bidirectional scans), then publishes
// the chunk's ready flag.  One workgroup per (chunk, batch*head), numbered in
// the order the state chain consumes the chunks.
//
// Every launcher, given `query`, fills it with the kernel's attributes
// (registers per lane, static LDS) instead of launching.
template <typename MT, int DK, int C>
hipError_t launch_prep(const ScanArgs& a, hipStream_t stream, hipFuncAttributes* query);

// Zeroes the n chunk-ready flags (before a concurrent preparation pass).
hipError_t launch_clear_ready(unsigned* ready, int64_t n, hipStream_t stream);

// Sequential inter-chunk state chain with the chunk outputs fused in.
// NT: 16-column value tiles per workgroup; BI: bidirectional (one workgroup
// per direction; the second visitor of a chunk adds the first one's readout,
// which it recognises against the pattern the preparation kernel filled the
// output with) instead of one direction (`rev_single` tells which).
// The state chain reads a chunk's prepared operands only after the chunk's
// ready flag is 1, so it may run concurrently with the preparation kernel.
template <typename MT, int DK, int C, int NT, bool BI>
hipError_t launch_chain(const ScanArgs& a, int rev_single, hipStream_t stream, hipFuncAttributes* query);

// Workgroups of a state-chain launch (one per value tile, direction and
// sequence; sequences padded to a multiple of eight).
inline int64_t chain_blocks(int64_t nbh, int dv, int NT, int dirs) { return (nbh + 7) / 8 * 8 * (dv / (16 * NT)) * dirs; }

// Frame-wise delta operator: per-frame products and inverses, the frame
// chain, and the readout, enqueued in that order on `stream`; ev (optional)
// receives events after the first and second kernels (ev[1], ev[2]).
template <typename MT, int DK, int DV>
hipError_t launch_vda(const VdaArgs& a, hipStream_t stream, hipEvent_t* ev);

}  // namespace gdn

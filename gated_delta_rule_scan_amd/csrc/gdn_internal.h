// Internal launch entry points of the libgdn kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_common.h"

namespace gdn {

// State-independent chunk quantities (triangular inverses, decayed q.k,
// per-token scales); for bidirectional scans, fills the output rows of its
// chunk with the "not written yet" pattern (a.zero_out, fp32 operands) or
// clears the chunk's combine flags (a.part_flags, bf16 operands); then
// publishes the chunk's ready flag.  One workgroup per (chunk, batch*head), numbered in
// the order the state chain consumes the chunks.
//
// Every launcher, given `query`, fills it with the kernel's attributes
// (registers per lane, static LDS) instead of launching.
template <typename MT, int DK, int C>
hipError_t launch_prep(const ScanArgs& a, hipStream_t stream, hipFuncAttributes* query);

// The same for 128-token chunks (C = 128): one 512-thread workgroup per
// (chunk, batch*head), the inverse blocked over fp32 tiles in LDS.
template <typename MT, int DK>
hipError_t launch_prep_wide(const ScanArgs& a, hipStream_t stream, hipFuncAttributes* query);

// Compute units of the current device (queried once per device; 256 on
// MI355X, also when the query fails).
int device_compute_units();

// Marks the n chunk-ready flags pending (1), before a concurrent preparation
// pass; the preparation kernel stores 0 once a chunk is ready.
hipError_t launch_clear_ready(unsigned* ready, int64_t n, hipStream_t stream);

// Sequential inter-chunk state chain with the chunk outputs fused in.
// NT: 16-column value tiles per workgroup; BI: bidirectional (one workgroup
// per direction; the second visitor of a chunk adds the first one's readout,
// which it recognises against the pattern the preparation kernel filled the
// output with) instead of one direction (`rev_single` tells which).
// With a.ready set, the state chain reads a chunk's prepared operands only
// once the chunk's ready flag is 0, so it may run concurrently with the
// preparation kernel.
template <typename MT, int DK, int C, int NT, bool BI>
hipError_t launch_chain(const ScanArgs& a, int rev_single, hipStream_t stream, hipFuncAttributes* query);

// The state chain for bf16 operands: NT chain waves each own 16 value columns
// of the state over every dk, NT readout waves compute the chunk outputs a
// step later; operands are staged by direct buffer-to-LDS loads.  Same
// arguments, grid and results contract as launch_chain<bf16, ...>, except
// that a bidirectional launch signals its partial readouts through
// a.part_flags (cleared by the preparation kernel, which must have finished).
// PREC: 0, bf16 operands throughout; 1, the readout's entry state also as
// its bf16 low parts (scans with the readout epilogue); 2, in addition the
// decayed q.k tile's low parts (a.pq_lo), added in the readouts of the
// directions that read before the token's own write (NT = 1 only).
template <int DK, int C, int NT, bool BI, int PREC>
hipError_t launch_column_chain(const ScanArgs& a, int rev_single, hipStream_t stream, hipFuncAttributes* query);

// The token scan's readout epilogue, in place on `out` ([rows, DV] fp32):
// out = norm_weight * o / sqrt(mean(o^2) + eps) * sigmoid(gate) per row.
template <typename MT, int DV>
hipError_t launch_epilogue(float* out, const void* gate, const float* norm_weight, float eps, int64_t rows,
                           hipStream_t stream);

// Workgroups of a state-chain launch (one per value tile, direction and
// sequence; sequences padded to a multiple of eight).
inline int64_t chain_blocks(int64_t nbh, int dv, int NT, int dirs) { return (nbh + 7) / 8 * 8 * (dv / (16 * NT)) * dirs; }

// Frame-wise delta operator: per-frame products and inverses, the frame
// chain, and the readout, enqueued in that order on `stream`; ev (optional)
// receives events after the first and second kernels (ev[1], ev[2]).
template <typename MT, int DK, int DV>
hipError_t launch_vda(const VdaArgs& a, hipStream_t stream, hipEvent_t* ev);

}  // namespace gdn

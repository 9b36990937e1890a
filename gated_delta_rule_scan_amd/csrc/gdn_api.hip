// libgdn C ABI: argument validation, workspace carving and kernel dispatch.
//
// Everything here is host code.  Validation finishes before anything is
// enqueued, so a rejected call leaves every buffer untouched; a valid call
// enqueues two kernels (chunk preparation, then the state chain) on the
// caller's stream and returns without synchronising.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "gdn.h"
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

struct Plan {
  int C;        // chunk length
  int NT;       // 16-column value tiles per chain workgroup (0: chosen at launch)
  int dirs;     // computed directions (slots)
  int fwd_on, rev_on;
  int64_t NC;   // chunks per sequence
  size_t mt;    // bytes per operand element
  WsLayout ws;
};

bool supported_dim(int64_t d) { return d == 64 || d == 128; }

// Compute units of the current device (cached per device; 256 on MI355X).
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int pick_tiles(int64_t nbh, int64_t dv, int dirs) {
  // A 32-wide value tile amortises the per-step fixed work of a chain (k
  // tile, triangles, barriers) over twice the columns.  That beats 16-wide
  // chains as soon as those would have to share compute units (measured on
  // MI355X: 1.4x for 384 16-wide chains on 256 units, even though the 192
  // wider chains leave a quarter of the units idle); with fewer chains than
  // units, the narrower tiles keep more units busy.
  if (nbh * dirs * (dv / 16) > compute_units()) return 2;
  return 1;
}

gdn_status_t make_plan(const gdn_problem_t* p, int32_t direction, Plan* pl) {
  if (!p) return GDN_ERR_INVALID_ARGUMENT;
  if (direction < GDN_DIR_FORWARD || direction > GDN_DIR_BIDIRECTIONAL) return GDN_ERR_INVALID_ARGUMENT;
  if (p->B < 1 || p->H < 1 || p->T < 0 || p->dk < 1 || p->dv < 1) return GDN_ERR_INVALID_ARGUMENT;
  if (p->reserved != 0) return GDN_ERR_INVALID_ARGUMENT;
  if (p->dtype != GDN_DTYPE_F32 && p->dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
  if (!supported_dim(p->dk) || !supported_dim(p->dv)) return GDN_ERR_UNSUPPORTED;
  if (p->B * p->H > 65535) return GDN_ERR_UNSUPPORTED;  // grid limit of the preparation kernel
  if (p->T > ((int64_t)1 << 31) / 2) return GDN_ERR_UNSUPPORTED;
  // every kernel addresses one (batch, head) sequence -- its rows interleaved
  // with the other heads' -- through 32-bit byte offsets
  if ((p->T + 64) * p->H * (p->dk > p->dv ? p->dk : p->dv) * 4 >= ((int64_t)1 << 32)) return GDN_ERR_UNSUPPORTED;
  const int C = p->chunk == 0 ? 64 : p->chunk;
  if (C != 32 && C != 64) return GDN_ERR_UNSUPPORTED;
  int NT = 0;  // 0: chosen at launch (any choice divides dv)
  if (p->dv_tile != 0) {
    if (p->dv_tile != 16 && p->dv_tile != 32) return GDN_ERR_UNSUPPORTED;
    NT = p->dv_tile / 16;
    if (p->dv % (16 * NT) != 0) return GDN_ERR_UNSUPPORTED;
  }
  pl->C = C;
  pl->NT = NT;
  pl->fwd_on = direction != GDN_DIR_REVERSE;
  pl->rev_on = direction != GDN_DIR_FORWARD;
  pl->dirs = pl->fwd_on + pl->rev_on;
  pl->NC = (p->T + C - 1) / C;
  pl->mt = p->dtype == GDN_DTYPE_BF16 ? 2 : 4;
  pl->ws = ws_layout(p->B * p->H, pl->NC, C, pl->dirs, pl->mt);
  return GDN_OK;
}

struct Range {
  uintptr_t lo, hi;
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

Range rng(const void* p, size_t bytes) {
  uintptr_t u = reinterpret_cast<uintptr_t>(p);
  return Range{u, p ? u + bytes : u};
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

typedef hipError_t (*prep_fn)(const ScanArgs&, hipStream_t);
typedef hipError_t (*chain_fn)(const ScanArgs&, int, hipStream_t);

template <typename MT>
prep_fn prep_for(int dk, int C) {
  if (dk == 64) return C == 32 ? launch_prep<MT, 64, 32> : launch_prep<MT, 64, 64>;
  return C == 32 ? launch_prep<MT, 128, 32> : launch_prep<MT, 128, 64>;
}

template <typename MT, int DK, int C>
chain_fn chain_for3(int NT, int dirs) {
  if (NT == 1) return dirs == 2 ? launch_chain<MT, DK, C, 1, true> : launch_chain<MT, DK, C, 1, false>;
  return dirs == 2 ? launch_chain<MT, DK, C, 2, true> : launch_chain<MT, DK, C, 2, false>;
}

template <typename MT>
chain_fn chain_for(int dk, int C, int NT, int dirs) {
  if (dk == 64) return C == 32 ? chain_for3<MT, 64, 32>(NT, dirs) : chain_for3<MT, 64, 64>(NT, dirs);
  return C == 32 ? chain_for3<MT, 128, 32>(NT, dirs) : chain_for3<MT, 128, 64>(NT, dirs);
}

}  // namespace
}  // namespace gdn

using namespace gdn;

extern "C" size_t gdn_workspace_bytes(const gdn_problem_t* p, int32_t direction) {
  Plan pl;
  if (make_plan(p, direction, &pl) != GDN_OK) return 0;
  return pl.ws.total;
}

extern "C" gdn_status_t gdn_forward(const gdn_problem_t* p, const void* q, const void* k, const void* v,
                                    const float* log_alpha, const float* beta, const float* state_in,
                                    float* state_out, float* out, int32_t direction) {
  Plan pl;
  gdn_status_t st = make_plan(p, direction, &pl);
  if (st != GDN_OK) return st;
  const int64_t B = p->B, T = p->T, H = p->H, dk = p->dk, dv = p->dv;
  const size_t es = pl.mt;
  const size_t n_qk = (size_t)(B * T * H * dk), n_v = (size_t)(B * T * H * dv);
  const size_t n_g = (size_t)(pl.dirs * B * T * H), n_s = (size_t)(pl.dirs * B * H * dv * dk);

  // required pointers and alignment
  if (T > 0) {
    if (!q || !k || !v || !log_alpha || !beta || !out) return GDN_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return GDN_ERR_INVALID_ARGUMENT;
    if (!aligned(log_alpha, 4) || !aligned(beta, 4)) return GDN_ERR_INVALID_ARGUMENT;
  }
  if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16))) return GDN_ERR_INVALID_ARGUMENT;
  const bool need_ws = T > 0;
  if (need_ws) {
    if (!p->workspace || !aligned(p->workspace, 256)) return GDN_ERR_INVALID_ARGUMENT;
    if (p->workspace_bytes < pl.ws.total) return GDN_ERR_WORKSPACE_TOO_SMALL;
  }

  // aliasing: outputs and workspace must not overlap anything else;
  // state_in == state_out (in-place carry) is the one allowed exception.
  const Range r_q = rng(q, n_qk * es), r_k = rng(k, n_qk * es), r_v = rng(v, n_v * es);
  const Range r_la = rng(log_alpha, n_g * 4), r_b = rng(beta, n_g * 4);
  const Range r_si = rng(state_in, n_s * 4), r_so = rng(state_out, n_s * 4);
  const Range r_o = rng(out, n_v * 4), r_ws = rng(need_ws ? p->workspace : nullptr, pl.ws.total);
  const Range ins[] = {r_q, r_k, r_v, r_la, r_b, r_si};
  for (const Range& r : ins) {
    if (overlap(r_o, r) || overlap(r_ws, r)) return GDN_ERR_INVALID_ARGUMENT;
  }
  for (int i = 0; i < 5; ++i)
    if (overlap(r_so, ins[i])) return GDN_ERR_INVALID_ARGUMENT;
  if (overlap(r_so, r_si) && state_in != state_out) return GDN_ERR_INVALID_ARGUMENT;
  if (overlap(r_o, r_so) || overlap(r_o, r_ws) || overlap(r_so, r_ws)) return GDN_ERR_INVALID_ARGUMENT;

  if (T == 0 && !state_out) return GDN_OK;  // nothing to compute or write

  hipStream_t stream = static_cast<hipStream_t>(p->stream);
  ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
  a.state_in = state_in; a.state_out = state_out; a.out = out;
  unsigned char* ws = static_cast<unsigned char*>(p->workspace);
  if (need_ws) {
    a.tri = ws + pl.ws.tri;
    a.pqk = ws + pl.ws.pqk;
    a.sc = reinterpret_cast<float4*>(ws + pl.ws.sc);
    a.pdg = reinterpret_cast<float*>(ws + pl.ws.pdg);
  }
  a.B = B; a.T = T; a.H = H; a.NC = pl.NC; a.dv = (int)dv;
  a.fwd_on = pl.fwd_on; a.rev_on = pl.rev_on; a.dirs = pl.dirs;
  a.zero_out = pl.dirs == 2;

  const bool bf = p->dtype == GDN_DTYPE_BF16;
  if (pl.NT == 0) pl.NT = pick_tiles(B * H, dv, pl.dirs);
  hipEvent_t* ev = static_cast<hipEvent_t*>(p->timing_events);
  hipError_t e = hipSuccess;
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return GDN_ERR_HIP;
  if (pl.NC > 0) {
    prep_fn pf = bf ? prep_for<bf16>((int)dk, pl.C) : prep_for<float>((int)dk, pl.C);
    e = pf(a, stream);
    if (e != hipSuccess) return GDN_ERR_HIP;
  }
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return GDN_ERR_HIP;
  // bidirectional: one workgroup per direction, readouts accumulated into
  // the output the preparation kernel zeroed; single direction: told whether
  // it runs in reverse
  chain_fn cf = bf ? chain_for<bf16>((int)dk, pl.C, pl.NT, pl.dirs)
                   : chain_for<float>((int)dk, pl.C, pl.NT, pl.dirs);
  if (!cf) return GDN_ERR_UNSUPPORTED;
  e = cf(a, direction == GDN_DIR_REVERSE ? 1 : 0, stream);
  if (e != hipSuccess) return GDN_ERR_HIP;
  if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return GDN_ERR_HIP;
  return GDN_OK;
}

extern "C" const char* gdn_status_string(int32_t s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported problem (dk, dv, chunk, tile or dtype)";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GDN_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

extern "C" const char* gdn_version(void) { return "libgdn 0.1.0 (gfx950)"; }

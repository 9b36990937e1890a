// libgdn C ABI: argument validation, workspace carving and kernel dispatch.
//
// Everything here is host code.  Validation finishes before anything is
// enqueued, so a rejected call leaves every buffer untouched; a valid call
// enqueues the chunk preparation and the state chain and returns without
// synchronising.  The two kernels run one after the other on the caller's
// stream, or -- when the device provably has room for a preparation
// workgroup beside every resident state-chain workgroup, and the stream is
// not being captured -- concurrently: the preparation pass on a library
// stream forked from and joined back to the caller's stream with events, the
// state chain on the caller's stream waiting chunk by chunk on the ready
// flags.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

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
  bool plo;     // the decayed q.k tile as hi + lo parts (exclusive readouts, bf16)
  WsLayout ws;
};

bool supported_dim(int64_t d) { return d == 64 || d == 128; }

int compute_units() { return device_compute_units(); }

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
  if ((p->options & ~(GDN_OPT_SERIAL | GDN_OPT_NO_ERASE | GDN_OPT_EXCLUSIVE_FORWARD | GDN_OPT_EXCLUSIVE_REVERSE |
                      GDN_OPT_TEST_NO_PREPARATION)) != 0)
    return GDN_ERR_INVALID_ARGUMENT;
  // the test option needs the ready-flag path, which the serial order does not take
  if ((p->options & GDN_OPT_TEST_NO_PREPARATION) && (p->options & GDN_OPT_SERIAL)) return GDN_ERR_INVALID_ARGUMENT;
  // the readout epilogue: a weight vector and a finite, non-negative eps
  if (p->gate && (!p->norm_weight || !(p->norm_eps >= 0.f) || !(p->norm_eps <= 3.4e38f))) return GDN_ERR_INVALID_ARGUMENT;
  if (p->dtype != GDN_DTYPE_F32 && p->dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
  if (!supported_dim(p->dk) || !supported_dim(p->dv)) return GDN_ERR_UNSUPPORTED;
  if (p->B * p->H > 65535) return GDN_ERR_UNSUPPORTED;  // grid limit of the preparation kernel
  if (p->T > ((int64_t)1 << 31) / 2) return GDN_ERR_UNSUPPORTED;
  // every kernel addresses one (batch, head) sequence -- its rows interleaved
  // with the other heads' -- through 32-bit byte offsets
  if ((p->T + 64) * p->H * (p->dk > p->dv ? p->dk : p->dv) * 4 >= ((int64_t)1 << 32)) return GDN_ERR_UNSUPPORTED;
  const int C = p->chunk == 0 ? 64 : p->chunk;
  if (C != 16 && C != 32 && C != 64 && C != 128) return GDN_ERR_UNSUPPORTED;
  const bool excl = (p->options & (GDN_OPT_EXCLUSIVE_FORWARD | GDN_OPT_EXCLUSIVE_REVERSE)) != 0;
  // 16- and 128-token chunks run the two-role chain for both operand types,
  // whose bf16 readout carries the entry state and P in bf16 only: the
  // exclusive readouts and the epilogue, which need their low parts, take 32-
  // or 64-token chunks
  if ((C == 16 || C == 128) && p->dtype == GDN_DTYPE_BF16 && (excl || p->gate)) return GDN_ERR_UNSUPPORTED;
  int NT = 0;  // 0: chosen at launch (any choice divides dv)
  if (p->dv_tile != 0) {
    if (p->dv_tile != 16 && p->dv_tile != 32) return GDN_ERR_UNSUPPORTED;
    NT = p->dv_tile / 16;
    if (p->dv % (16 * NT) != 0) return GDN_ERR_UNSUPPORTED;
  }
  // fp32 operands with dk = 128 fit 16-column tiles only at 128-token chunks
  const bool narrow = C == 128 && p->dtype == GDN_DTYPE_F32 && p->dk == 128;
  if (narrow) {
    if (NT == 2) return GDN_ERR_UNSUPPORTED;
    NT = 1;
  }
  pl->C = C;
  pl->NT = NT;
  pl->fwd_on = direction != GDN_DIR_REVERSE;
  pl->rev_on = direction != GDN_DIR_FORWARD;
  pl->dirs = pl->fwd_on + pl->rev_on;
  pl->NC = (p->T + C - 1) / C;
  pl->mt = p->dtype == GDN_DTYPE_BF16 ? 2 : 4;
  // exclusive readouts on bf16 operands carry the decayed q.k tile as hi + lo parts
  pl->plo = p->dtype == GDN_DTYPE_BF16 && excl;
  // (and the entry state's low parts: their exchange fits 16-column tiles only)
  if (pl->plo) {
    if (pl->NT == 2) return GDN_ERR_UNSUPPORTED;
    pl->NT = 1;
  }
  pl->ws = ws_layout(p->B * p->H, pl->NC, C, pl->dirs, pl->mt, p->dv, pl->plo);
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

typedef hipError_t (*prep_fn)(const ScanArgs&, hipStream_t, hipFuncAttributes*);
typedef hipError_t (*chain_fn)(const ScanArgs&, int, hipStream_t, hipFuncAttributes*);

// ---- concurrent preparation ----
// Per device: the library's side stream (default priority) and the fork and
// join events, created on first use and kept for the life of the process.
// One mutex serialises the enqueue sequences that share them.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];

bool side_stream(int dev, SideStream** out) {
  if (dev < 0 || dev >= 64) return false;
  SideStream& s = g_side[dev];
  if (!s.stream) {
    if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess) return false;
    if (hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess) return false;
  }
  *out = &s;
  return true;
}

// Whether the preparation pass runs concurrently with the state chain.
//
// Worth it only when the chain leaves compute units free and is long enough
// to hide the pass: preparation workgroups beside the chain slow it down
// (they share L2 and the memory path).  Measured on MI355X with the bf16
// column chain, which prefetches a chunk's prepared tiles into L2 once its
// ready flag reads ready: 720p causal (128 chain workgroups on 256 units,
// 1182 chunks) 1.60 ms concurrent against 1.71 ms serial; the streaming 480p
// frames (96 workgroups, 25 chunks) 0.060 against 0.045 ms per frame; 480p
// and 720p bidirectional hold every unit and run serial.  So the overlap is
// taken when the chain holds at most half of the units and has at least 128
// chunks (the column chain), or at most a quarter of the units and 16 chunks
// (the two-role chain, which has no such prefetch).  (Bidirectional
// column-chain scans always run serial; see forward_impl.)
//
// Safe because the chain waits only for chunks the preparation pass
// publishes, and a preparation workgroup can always be scheduled: at most
// half of the compute units hold a chain workgroup, and the preparation,
// which never waits, is kept off those units beside a 16-column chain (it
// then asks for more LDS than such a unit has left).  The preparation pass
// is enqueued first, so a device that runs the two streams one after the
// other still finishes it before the chain starts.
bool may_overlap(int64_t chain_wgs, int64_t NC, bool column) {
  if (column) return NC >= 128 && 2 * chain_wgs <= (int64_t)compute_units();
  constexpr int64_t kMinChunks = 16;  // below this the fork/join costs more than it hides
  return NC >= kMinChunks && 4 * chain_wgs <= (int64_t)compute_units();
}

// Whether `stream` is being captured into a graph (any capture mode).  A
// failed query counts as capturing, which only selects the serial order.
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return true;
  return st != hipStreamCaptureStatusNone;
}

template <typename MT>
prep_fn prep_for(int dk, int C) {
  if (C == 128) return dk == 64 ? launch_prep_wide<MT, 64> : launch_prep_wide<MT, 128>;
  if (C == 16) return dk == 64 ? launch_prep<MT, 64, 16> : launch_prep<MT, 128, 16>;
  if (dk == 64) return C == 32 ? launch_prep<MT, 64, 32> : launch_prep<MT, 64, 64>;
  return C == 32 ? launch_prep<MT, 128, 32> : launch_prep<MT, 128, 64>;
}

template <typename MT, int DK, int C>
chain_fn chain_for3(int NT, int dirs) {
  if (NT == 1) return dirs == 2 ? launch_chain<MT, DK, C, 1, true> : launch_chain<MT, DK, C, 1, false>;
  return dirs == 2 ? launch_chain<MT, DK, C, 2, true> : launch_chain<MT, DK, C, 2, false>;
}

template <int DK, int C, int PREC>
chain_fn column_chain_for4(int NT, int dirs) {
  if (NT == 1) return dirs == 2 ? launch_column_chain<DK, C, 1, true, PREC> : launch_column_chain<DK, C, 1, false, PREC>;
  return dirs == 2 ? launch_column_chain<DK, C, 2, true, PREC> : launch_column_chain<DK, C, 2, false, PREC>;
}

template <int DK, int C>
chain_fn column_chain_for3(int NT, int dirs, int prec) {
  if (prec == 2) {  // 16-column tiles only
    if (NT != 1) return nullptr;
    return dirs == 2 ? launch_column_chain<DK, C, 1, true, 2> : launch_column_chain<DK, C, 1, false, 2>;
  }
  return prec == 1 ? column_chain_for4<DK, C, 1>(NT, dirs) : column_chain_for4<DK, C, 0>(NT, dirs);
}

// bf16 operands: the column-owning chain; fp32 operands, and 16- and
// 128-token chunks of either type: the two-role chain
template <typename MT>
chain_fn chain_for(int dk, int C, int NT, int dirs, int prec) {
  if (C == 16) return dk == 64 ? chain_for3<MT, 64, 16>(NT, dirs) : chain_for3<MT, 128, 16>(NT, dirs);
  if (C == 128) {
    if (dk == 64) return chain_for3<MT, 64, 128>(NT, dirs);
    if constexpr (sizeof(MT) == 4) {
      if (NT != 1) return nullptr;
      return dirs == 2 ? launch_chain<float, 128, 128, 1, true> : launch_chain<float, 128, 128, 1, false>;
    } else {
      return chain_for3<MT, 128, 128>(NT, dirs);
    }
  }
  if constexpr (sizeof(MT) == 2) {
    if (dk == 64) return C == 32 ? column_chain_for3<64, 32>(NT, dirs, prec) : column_chain_for3<64, 64>(NT, dirs, prec);
    return C == 32 ? column_chain_for3<128, 32>(NT, dirs, prec) : column_chain_for3<128, 64>(NT, dirs, prec);
  } else {
    if (dk == 64) return C == 32 ? chain_for3<MT, 64, 32>(NT, dirs) : chain_for3<MT, 64, 64>(NT, dirs);
    return C == 32 ? chain_for3<MT, 128, 32>(NT, dirs) : chain_for3<MT, 128, 64>(NT, dirs);
  }
}

}  // namespace
}  // namespace gdn

using namespace gdn;

namespace gdn {

int device_compute_units() {
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

}  // namespace gdn

extern "C" size_t gdn_workspace_bytes(const gdn_problem_t* p, int32_t direction) {
  Plan pl;
  if (make_plan(p, direction, &pl) != GDN_OK) return 0;
  return pl.ws.total;
}

namespace gdn {
namespace {

// The whole call with an explicit workspace (ws, ws_bytes); `serial_only`
// keeps both kernels on the caller's stream.
gdn_status_t forward_impl(const gdn_problem_t* p, void* ws_ptr, size_t ws_bytes, bool serial_only, const void* q,
                          const void* k, const void* v, const float* log_alpha, const float* beta,
                          const float* state_in, float* state_out, float* out, int32_t direction) {
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
  if (p->gate && (!aligned(p->gate, 16) || !aligned(p->norm_weight, 16))) return GDN_ERR_INVALID_ARGUMENT;
  const bool need_ws = T > 0;
  if (need_ws) {
    if (!ws_ptr || !aligned(ws_ptr, 256)) return GDN_ERR_INVALID_ARGUMENT;
    if (ws_bytes < pl.ws.total) return GDN_ERR_WORKSPACE_TOO_SMALL;
  }

  // aliasing: outputs and workspace must not overlap anything else;
  // state_in == state_out (in-place carry) is the one allowed exception.
  const Range r_q = rng(q, n_qk * es), r_k = rng(k, n_qk * es), r_v = rng(v, n_v * es);
  const Range r_la = rng(log_alpha, n_g * 4), r_b = rng(beta, n_g * 4);
  const Range r_si = rng(state_in, n_s * 4), r_so = rng(state_out, n_s * 4);
  const Range r_o = rng(out, n_v * 4), r_ws = rng(need_ws ? ws_ptr : nullptr, pl.ws.total);
  const Range r_g = rng(p->gate, n_v * es), r_nw = rng(p->gate ? p->norm_weight : nullptr, (size_t)dv * 4);
  const Range ins[] = {r_q, r_k, r_v, r_la, r_b, r_g, r_nw, r_si};
  for (const Range& r : ins) {
    if (overlap(r_o, r) || overlap(r_ws, r)) return GDN_ERR_INVALID_ARGUMENT;
  }
  for (int i = 0; i < 7; ++i)
    if (overlap(r_so, ins[i])) return GDN_ERR_INVALID_ARGUMENT;
  if (overlap(r_so, r_si) && state_in != state_out) return GDN_ERR_INVALID_ARGUMENT;
  if (overlap(r_o, r_so) || overlap(r_o, r_ws) || overlap(r_so, r_ws)) return GDN_ERR_INVALID_ARGUMENT;

  if (T == 0 && !state_out) return GDN_OK;  // nothing to compute or write

  hipStream_t stream = static_cast<hipStream_t>(p->stream);
  ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
  a.state_in = state_in; a.state_out = state_out; a.out = out;
  unsigned char* ws = static_cast<unsigned char*>(ws_ptr);
  if (need_ws) {
    a.tri = ws + pl.ws.tri;
    a.pqk = ws + pl.ws.pqk;
    a.sc = reinterpret_cast<float4*>(ws + pl.ws.sc);
    a.pdg = reinterpret_cast<float*>(ws + pl.ws.pdg);
  }
  a.B = B; a.T = T; a.H = H; a.NC = pl.NC; a.dv = (int)dv;
  a.fwd_on = pl.fwd_on; a.rev_on = pl.rev_on; a.dirs = pl.dirs;
  const bool bf = p->dtype == GDN_DTYPE_BF16;
  // bidirectional combine: the two-role chain (fp32 operands, 128-token
  // chunks) recognises an unwritten partial by the preparation kernel's fill
  // of `out`; the column chain by per-chunk flags that the preparation kernel
  // clears
  const bool column = bf && pl.C != 128 && pl.C != 16;
  a.zero_out = pl.dirs == 2 && !column;
  if (pl.dirs == 2 && column && need_ws) a.part_flags = reinterpret_cast<unsigned*>(ws + pl.ws.pfl);
  if (pl.plo && need_ws) a.pq_lo = ws + pl.ws.pql;
  a.erase = (p->options & GDN_OPT_NO_ERASE) ? 0 : 1;
  a.excl_fwd = (p->options & GDN_OPT_EXCLUSIVE_FORWARD) ? 1 : 0;
  a.excl_rev = (p->options & GDN_OPT_EXCLUSIVE_REVERSE) ? 1 : 0;

  if (pl.NT == 0) pl.NT = pick_tiles(B * H, dv, pl.dirs);
  // bidirectional: one workgroup per direction, readouts accumulated into
  // the output the preparation kernel filled; single direction: told whether
  // it runs in reverse
  chain_fn cf = bf ? chain_for<bf16>((int)dk, pl.C, pl.NT, pl.dirs, pl.plo ? 2 : (p->gate ? 1 : 0))
                   : chain_for<float>((int)dk, pl.C, pl.NT, pl.dirs, 0);
  prep_fn pf = bf ? prep_for<bf16>((int)dk, pl.C) : prep_for<float>((int)dk, pl.C);
  if (!cf || !pf) return GDN_ERR_UNSUPPORTED;
  const int rev_single = direction == GDN_DIR_REVERSE ? 1 : 0;
  hipEvent_t* ev = static_cast<hipEvent_t*>(p->timing_events);
  auto mark = [&](int i, hipStream_t st) { return !ev || hipEventRecord(ev[i], st) == hipSuccess; };

  // the readout epilogue, after the chain on `stream`
  auto epilogue = [&]() -> bool {
    if (!p->gate || T == 0) return true;
    const int64_t rows = B * T * H;
    hipError_t e;
    if (bf) e = dv == 64 ? launch_epilogue<bf16, 64>(out, p->gate, p->norm_weight, p->norm_eps, rows, stream)
                         : launch_epilogue<bf16, 128>(out, p->gate, p->norm_weight, p->norm_eps, rows, stream);
    else e = dv == 64 ? launch_epilogue<float, 64>(out, p->gate, p->norm_weight, p->norm_eps, rows, stream)
                      : launch_epilogue<float, 128>(out, p->gate, p->norm_weight, p->norm_eps, rows, stream);
    return e == hipSuccess;
  };
  const bool skip_prep = (p->options & GDN_OPT_TEST_NO_PREPARATION) != 0;
  if (skip_prep && pl.NC > 0) {
    // flags marked pending and never cleared: the chain's bounded waits expire
    a.ready = reinterpret_cast<unsigned*>(ws + pl.ws.rdy);
    if (launch_clear_ready(a.ready, B * H * pl.NC, stream) != hipSuccess) return GDN_ERR_HIP;
    if (!mark(0, stream) || !mark(1, stream) || !mark(2, stream)) return GDN_ERR_HIP;
    if (cf(a, rev_single, stream, nullptr) != hipSuccess || !mark(3, stream)) return GDN_ERR_HIP;
    return epilogue() ? GDN_OK : GDN_ERR_HIP;
  }
  // Under stream capture the two kernels always run one after the other: a
  // graph orders its nodes only by their dependencies, so nothing would make
  // the preparation node start while the chain node waits on its flags, and
  // no library stream or event may be created or joined into a capture.
  // A bidirectional bf16 scan always takes the serial order: its chain reads
  // the combine flags ahead of the chunk-ready flags, so they must be clear
  // before it starts.
  const bool concurrent = pl.NC > 0 && !serial_only && !(p->options & GDN_OPT_SERIAL) && !capturing(stream) &&
                          !a.part_flags && may_overlap(chain_blocks(B * H, (int)dv, pl.NT, pl.dirs), pl.NC, column);
  if (concurrent) {
    int dev = 0;
    SideStream* side = nullptr;
    std::lock_guard<std::mutex> lock(g_side_mu);
    if (hipGetDevice(&dev) != hipSuccess || !side_stream(dev, &side)) return GDN_ERR_HIP;
    a.ready = reinterpret_cast<unsigned*>(ws + pl.ws.rdy);
    // the flags start as pending before either kernel can see them; the
    // side stream forks after that, and the preparation pass is enqueued first
    if (launch_clear_ready(a.ready, B * H * pl.NC, stream) != hipSuccess) return GDN_ERR_HIP;
    if (hipEventRecord(side->fork, stream) != hipSuccess) return GDN_ERR_HIP;
    if (hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess) return GDN_ERR_HIP;
    if (!mark(0, side->stream) || pf(a, side->stream, nullptr) != hipSuccess || !mark(1, side->stream))
      return GDN_ERR_HIP;
    if (hipEventRecord(side->join, side->stream) != hipSuccess) return GDN_ERR_HIP;
    if (!mark(2, stream) || cf(a, rev_single, stream, nullptr) != hipSuccess || !mark(3, stream)) return GDN_ERR_HIP;
    if (hipStreamWaitEvent(stream, side->join, 0) != hipSuccess) return GDN_ERR_HIP;
    return epilogue() ? GDN_OK : GDN_ERR_HIP;
  }
  // one after the other on the caller's stream (no flags: a.ready stays null)
  if (!mark(0, stream)) return GDN_ERR_HIP;
  if (pl.NC > 0 && pf(a, stream, nullptr) != hipSuccess) return GDN_ERR_HIP;
  if (!mark(1, stream) || !mark(2, stream)) return GDN_ERR_HIP;
  if (cf(a, rev_single, stream, nullptr) != hipSuccess) return GDN_ERR_HIP;
  if (!mark(3, stream)) return GDN_ERR_HIP;
  return epilogue() ? GDN_OK : GDN_ERR_HIP;
}

// ---- the fixed device scratch of gdn_forward_noalloc ----
// Each device that loads the library holds its own copy of this array until
// the process ends.  Host code never passes the array's name to a kernel (in
// host code it is only a stand-in for the symbol): it uses the device address
// returned by hipGetSymbolAddress, looked up once per device with that device
// current.
constexpr size_t kScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

// Device address of the current device's scratch (nullptr on failure).
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace gdn

extern "C" gdn_status_t gdn_forward(const gdn_problem_t* p, const void* q, const void* k, const void* v,
                                    const float* log_alpha, const float* beta, const float* state_in,
                                    float* state_out, float* out, int32_t direction) {
  if (!p) return GDN_ERR_INVALID_ARGUMENT;
  return forward_impl(p, p->workspace, p->workspace_bytes, false, q, k, v, log_alpha, beta, state_in, state_out, out,
                      direction);
}

extern "C" gdn_status_t gdn_forward_noalloc(const gdn_problem_t* p, const void* q, const void* k, const void* v,
                                            const float* log_alpha, const float* beta, const float* state_in,
                                            float* state_out, float* out, int32_t direction) {
  if (!p) return GDN_ERR_INVALID_ARGUMENT;
  Plan pl;
  gdn_status_t st = make_plan(p, direction, &pl);
  if (st != GDN_OK) return st;
  // argument errors first (the rest of the checks follow in forward_impl)
  if (p->T > 0 && (!q || !k || !v || !log_alpha || !beta || !out)) return GDN_ERR_INVALID_ARGUMENT;
  if (p->T > 0 && pl.ws.total > kScratchBytes) return GDN_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (p->T > 0 && !(ws = scratch_address())) return GDN_ERR_HIP;
  return forward_impl(p, ws, kScratchBytes, true, q, k, v, log_alpha, beta, state_in, state_out, out, direction);
}

// ---- frame-wise delta operator ----
namespace gdn {
namespace {

typedef hipError_t (*vda_fn)(const VdaArgs&, hipStream_t, hipEvent_t*);

template <typename MT>
vda_fn vda_for(int64_t dk, int64_t dv) {
  if (dk == 64) return dv == 64 ? launch_vda<MT, 64, 64> : launch_vda<MT, 64, 128>;
  return dv == 64 ? launch_vda<MT, 128, 64> : launch_vda<MT, 128, 128>;
}

gdn_status_t vda_plan(const gdn_vda_problem_t* p, int32_t direction, int* dirs, int64_t* NF, VdaLayout* L) {
  if (!p) return GDN_ERR_INVALID_ARGUMENT;
  if (direction < GDN_DIR_FORWARD || direction > GDN_DIR_BIDIRECTIONAL) return GDN_ERR_INVALID_ARGUMENT;
  if (p->B < 1 || p->H < 1 || p->T < 0 || p->dk < 1 || p->dv < 1 || p->frame < 1) return GDN_ERR_INVALID_ARGUMENT;
  if ((p->options & ~GDN_VDA_OPT_ADDITIVE) != 0 || p->readout_lag < 0) return GDN_ERR_INVALID_ARGUMENT;
  if (p->gate && (!p->norm_weight || !(p->norm_eps >= 0.f) || !(p->norm_eps <= 3.4e38f))) return GDN_ERR_INVALID_ARGUMENT;
  if (p->dtype != GDN_DTYPE_F32 && p->dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
  if (!supported_dim(p->dk) || !supported_dim(p->dv)) return GDN_ERR_UNSUPPORTED;
  if (p->T > ((int64_t)1 << 31) / 2) return GDN_ERR_UNSUPPORTED;
  if ((p->T + 64) * p->H * (p->dk > p->dv ? p->dk : p->dv) * 4 >= ((int64_t)1 << 32)) return GDN_ERR_UNSUPPORTED;
  *dirs = direction == GDN_DIR_BIDIRECTIONAL ? 2 : 1;
  *NF = (p->T + p->frame - 1) / p->frame;
  // grid sizes: frame kernel (padded to groups of eight per direction) and
  // readout (runs of up to eight 64-token blocks per frame)
  const int64_t BH = p->B * p->H, nblk = (p->frame + 63) / 64;
  if (2 * ((BH * *NF + 7) / 8) * 8 > ((int64_t)1 << 31) - 1) return GDN_ERR_UNSUPPORTED;
  if (BH * *NF * ((nblk + 7) / 8) > ((int64_t)1 << 31) - 1) return GDN_ERR_UNSUPPORTED;
  *L = vda_layout(p->B * p->H, *NF, *dirs, p->dk, p->dv);
  return GDN_OK;
}

}  // namespace
}  // namespace gdn

extern "C" size_t gdn_vda_workspace_bytes(const gdn_vda_problem_t* p, int32_t direction) {
  int dirs = 0;
  int64_t NF = 0;
  VdaLayout L;
  if (vda_plan(p, direction, &dirs, &NF, &L) != GDN_OK || p->T == 0) return 0;
  return L.total;
}

extern "C" gdn_status_t gdn_vda_forward(const gdn_vda_problem_t* p, const void* q, const void* k, const void* v,
                                        const float* log_alpha, const float* beta, const float* state_in,
                                        float* state_out, float* out, int32_t direction) {
  int dirs = 0;
  int64_t NF = 0;
  VdaLayout L;
  gdn_status_t st = vda_plan(p, direction, &dirs, &NF, &L);
  if (st != GDN_OK) return st;
  const int64_t B = p->B, T = p->T, H = p->H, dk = p->dk, dv = p->dv;
  const size_t es = p->dtype == GDN_DTYPE_BF16 ? 2 : 4;
  const size_t n_qk = (size_t)(B * T * H * dk), n_v = (size_t)(B * T * H * dv);
  const size_t n_la = (size_t)(dirs * B * NF * H), n_b = (size_t)(dirs * B * T * H), n_s = (size_t)(dirs * B * H * dv * dk);
  if (T > 0) {
    if (!q || !k || !v || !log_alpha || !beta || !out) return GDN_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return GDN_ERR_INVALID_ARGUMENT;
    if (!aligned(log_alpha, 4) || !aligned(beta, 4)) return GDN_ERR_INVALID_ARGUMENT;
    if (!p->workspace || !aligned(p->workspace, 256)) return GDN_ERR_INVALID_ARGUMENT;
    if (p->workspace_bytes < L.total) return GDN_ERR_WORKSPACE_TOO_SMALL;
  }
  if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16))) return GDN_ERR_INVALID_ARGUMENT;
  if (p->gate && (!aligned(p->gate, 16) || !aligned(p->norm_weight, 16))) return GDN_ERR_INVALID_ARGUMENT;
  const Range r_q = rng(q, n_qk * es), r_k = rng(k, n_qk * es), r_v = rng(v, n_v * es);
  const Range r_la = rng(log_alpha, n_la * 4), r_b = rng(beta, n_b * 4);
  const Range r_si = rng(state_in, n_s * 4), r_so = rng(state_out, n_s * 4);
  const Range r_o = rng(out, n_v * 4), r_ws = rng(T > 0 ? p->workspace : nullptr, L.total);
  const Range r_g = rng(p->gate, n_v * es), r_nw = rng(p->gate ? p->norm_weight : nullptr, (size_t)dv * 4);
  const Range ins[] = {r_q, r_k, r_v, r_la, r_b, r_g, r_nw, r_si};
  for (const Range& r : ins)
    if (overlap(r_o, r) || overlap(r_ws, r)) return GDN_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 7; ++i)
    if (overlap(r_so, ins[i])) return GDN_ERR_INVALID_ARGUMENT;
  if (overlap(r_so, r_si) && state_in != state_out) return GDN_ERR_INVALID_ARGUMENT;
  if (overlap(r_o, r_so) || overlap(r_o, r_ws) || overlap(r_so, r_ws)) return GDN_ERR_INVALID_ARGUMENT;
  if (T == 0 && !state_out) return GDN_OK;

  VdaArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
  a.state_in = state_in; a.state_out = state_out; a.out = out;
  unsigned char* ws = static_cast<unsigned char*>(p->workspace);
  if (T > 0) {
    a.minv = reinterpret_cast<float*>(ws + L.minv);
    a.bmat = reinterpret_cast<float*>(ws + L.bmat);
    a.sfr = reinterpret_cast<float*>(ws + L.sfr);
  }
  a.B = B; a.T = T; a.H = H; a.NF = NF; a.frame = p->frame; a.dv = (int)dv;
  a.dirs = dirs;
  a.fwd_on = direction != GDN_DIR_REVERSE;
  a.rev_on = direction != GDN_DIR_FORWARD;
  a.additive = (p->options & GDN_VDA_OPT_ADDITIVE) != 0;
  a.lag = p->readout_lag < NF ? p->readout_lag : (int)(NF < 1 ? 1 : NF);  // NF or more: only initial states
  a.gate = p->gate;
  a.norm_weight = p->gate ? p->norm_weight : nullptr;
  a.norm_eps = p->norm_eps;
  hipStream_t stream = static_cast<hipStream_t>(p->stream);
  hipEvent_t* ev = static_cast<hipEvent_t*>(p->timing_events);
  vda_fn fn = p->dtype == GDN_DTYPE_BF16 ? vda_for<bf16>(dk, dv) : vda_for<float>(dk, dv);
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return GDN_ERR_HIP;
  if (fn(a, stream, ev) != hipSuccess) return GDN_ERR_HIP;
  if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return GDN_ERR_HIP;
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

// Shared device helpers for the libgdn kernels (gfx950 / CDNA4).
//
// Matrix-core fragments.  Every product in the chunked scan is issued as
// 16x16 output tiles with a contraction slice of 32:
//   * bf16 operands: one v_mfma_f32_16x16x32_bf16;
//   * fp32 operands: eight v_mfma_f32_16x16x4_f32.
// Both use the same lane layout (checked on gfx950):
//   A (16 x 32, row-major source M[row][k]): lane l holds M[l%16][8*(l/16) .. +7]
//   B (32 x 16, given transposed as Mt[col][k]): lane l holds Mt[l%16][8*(l/16) .. +7]
//   D (16 x 16, fp32): lane l holds D[4*(l/16) + i][l%16], i = 0..3
// For fp32 the eight k = 4 instructions take element j of every lane in
// instruction j; the contraction is a sum over all 32 k, so pairing the same
// (lane group, slot) of A and B gives the full product regardless of which
// hardware k index a slot lands on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNormEps = 1e-6f;  // q^ = q / max(|q|, eps)

template <typename MT>
struct Mma;

template <>
struct Mma<bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const bf16* p) {  // 16-byte aligned
    return *reinterpret_cast<const bf16x8*>(p);
  }
  static __device__ __forceinline__ frag zero() {
    frag z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
    return z;
  }
  static __device__ __forceinline__ float get(const frag& f, int e) { return (float)f[e]; }
  static __device__ __forceinline__ void set(frag& f, int e, float x) { f[e] = (bf16)x; }
  static __device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {  // 8-byte aligned
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *reinterpret_cast<bf16x4*>(p) = v;
  }
};

template <>
struct Mma<float> {
  struct frag {
    f32x4 lo, hi;
  };
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ frag load(const float* p) {  // 16-byte aligned
    frag f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f;
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
    f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
    f.hi = f.lo;
    return f;
  }
  static __device__ __forceinline__ float get(const frag& f, int e) { return e < 4 ? f.lo[e] : f.hi[e - 4]; }
  static __device__ __forceinline__ void set(frag& f, int e, float x) {
    if (e < 4) f.lo[e] = x; else f.hi[e - 4] = x;
  }
  static __device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {  // 16-byte aligned
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  }
};

// ---- raw buffer access ----------------------------------------------------
// Out-of-range loads return zero and out-of-range stores are dropped, so
// partial chunks need neither clamping nor branches.
// Word 3 of a gfx9 buffer resource for raw (unstructured) access with 32-bit
// elements; the hardware bounds every access by num_records bytes.
constexpr int kRawBufferWord3 = 0x00020000;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

__device__ __forceinline__ f32x4 bload16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  f32x4 f;
  __builtin_memcpy(&f, &v, 16);
  return f;
}

__device__ __forceinline__ float bload4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// s_waitcnt immediate that waits for every vector memory access of the
// wave (vmcnt 0; the other counters at their maxima)
constexpr int kWaitVmem = 0x0F70;

__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, f32x4 x) {
  u32x4 v;
  __builtin_memcpy(&v, &x, 16);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// Stores with the agent-scope cache policy (sc1): written through this XCD's
// L2 cache, so once the store counter has drained they are visible to every
// XCD of the device without a cache write-back.
constexpr int kAgentScope = 16;
__device__ __forceinline__ void bstore16_agent(rsrc_t r, uint32_t off, f32x4 x) {
  u32x4 v;
  __builtin_memcpy(&v, &x, 16);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kAgentScope);
}
__device__ __forceinline__ void bstore8_agent(rsrc_t r, uint32_t off, uint32_t lo, uint32_t hi) {
  typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, r, (int)off, 0, kAgentScope);
}
__device__ __forceinline__ void bstore4_agent(rsrc_t r, uint32_t off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), r, (int)off, 0, kAgentScope);
}
__device__ __forceinline__ void bstore4u_agent(rsrc_t r, uint32_t off, uint32_t x) {
  __builtin_amdgcn_raw_buffer_store_b32((int)x, r, (int)off, 0, kAgentScope);
}

// Workspace stores of a preparation pass: agent scope when the state chain
// may read them while the pass still runs (the concurrent order, which
// publishes each chunk with a ready flag), else the default policy for large
// passes (the chain starts after the pass has ended, and a plain store
// completes sooner: 480p bidirectional preparation 0.208 -> 0.189 ms,
// measured) but agent scope for small ones (whose time the write-back of
// dirty lines at the end of the kernel then dominates: a 1560-token
// streaming frame's pass 12.0 us with agent-scope stores, 13.9 us without).
// `agent` is uniform across the workgroup.
__device__ __forceinline__ void bstore16_ws(bool agent, rsrc_t r, uint32_t off, f32x4 x) {
  if (agent) bstore16_agent(r, off, x);
  else bstore16(r, off, x);
}
__device__ __forceinline__ void bstore8_ws(bool agent, rsrc_t r, uint32_t off, uint32_t lo, uint32_t hi) {
  typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
  if (agent) bstore8_agent(r, off, lo, hi);
  else __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore4_ws(bool agent, rsrc_t r, uint32_t off, float x) {
  if (agent) bstore4_agent(r, off, x);
  else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), r, (int)off, 0, 0);
}

// Every NaN replaced by the canonical quiet NaN.  A bidirectional scan's
// first visitor stores its readout through this, so its stores can never
// carry the all-ones "not written yet" pattern, whatever NaN payload an
// input held.
__device__ __forceinline__ f32x4 canonical_nans(f32x4 o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = o[i] != o[i] ? __builtin_nanf("") : o[i];
  return o;
}

// A matrix-core fragment (8 consecutive elements) at byte offset `off`.
template <typename MT>
__device__ __forceinline__ typename Mma<MT>::frag bload_frag(rsrc_t r, uint32_t off) {
  typename Mma<MT>::frag f;
  if constexpr (sizeof(MT) == 2) {
    const f32x4 v = bload16(r, off);
    __builtin_memcpy(&f, &v, 16);
  } else {
    f.lo = bload16(r, off);
    f.hi = bload16(r, off + 16);
  }
  return f;
}

// ---- transposed bf16 operands from row-major LDS tiles ----
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// ds_read_b64_tr_b16 transposes within each 16-lane group: lane i receives
// res[i][e] = src[4e + i/4][i % 4], where src[s] is the four consecutive bf16
// at source lane s's address (lane mapping checked on gfx950).
__device__ __forceinline__ v4s lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(const_cast<void*>(p)));
}

// Transposed k fragment for the state update, read from a row-major bf16 k
// tile in LDS.  The A operand (m = dk row dk0 + l16, k = 32 tokens from tok0)
// holds, in lane (l16, g4), k[tok0 + 8 g4 + j][dk0 + l16] for j = 0..7.
// Source lane s therefore points at k[tok + s/4][dk0 + 4 (s % 4)]; two reads
// give j = 0..3 and j = 4..7.
__device__ __forceinline__ bf16x8 load_kt_frag(const bf16* krow, int kp, int tok0, int dk0, int l16, int g4) {
  const int o0 = (tok0 + 8 * g4 + (l16 >> 2)) * kp + dk0 + 4 * (l16 & 3);
  const v4s lo = lds_read_tr16(krow + o0);
  const v4s hi = lds_read_tr16(krow + o0 + 4 * kp);
  bf16x8 r;
  __builtin_memcpy(&r, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi, 8);
  return r;
}

// ---------------------------------------------------------------------------
// Workspace layout (per problem; NBH = B*H chunk chains, NC chunks each,
// dirs = number of computed directions):
//   tri  [NBH*NC][C][C]  MT : strictly-lower part = forward (I+L)^{-1},
//                             strictly-upper part = reverse (I+L)^{-1}
//   pqk  [NBH*NC][C][C]  MT : decayed q^.k^ with the self terms q^_t.k^_t on
//                             the diagonal; strictly-lower part = forward,
//                             strictly-upper part = reverse
//   sc   [dirs][NBH*NC][C] float4 : {beta, e^g rk, e^g rq, e^(gn-g) rk}
//   pdg  [dirs][NBH*NC][PDS] float : e^(gn) (the chunk's total decay) and
//                             three zeros, then per token the part of the
//                             self term q^_t.k^_t that the operand type of
//                             pqk drops (x - MT(x); zero for fp32 operands)
//                             (C + 4 floats: whole 16-byte pieces), padded to
//                             PDS = pdg_stride(C) floats so that no 128-byte
//                             cache line holds two chunks' records
//   rdy  [NBH][NC] uint32 : per-chunk ready flags of the concurrent
//                             preparation: a small kernel marks every chunk 1
//                             (pending), the preparation kernel stores 0 once
//                             the chunk's outputs (and its output fill) are in
//                             place, and the state chain waits for 0
//   pfl  [NBH][NC][dv/16] uint32 : bidirectional scans on bf16 operands: per
//                             chunk and 16 output columns, 1 once the first
//                             visitor's readout (the partial the second
//                             visitor adds) is in `out`; the preparation
//                             kernel clears the chunk's flags
//   pql  [NBH*NC][C][C]  bf16 : exclusive readouts on bf16 operands: the
//                             part of each strict entry of pqk that bf16
//                             drops (x - bf16(x)); else absent
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t tri, pqk, sc, pdg, rdy, pfl, pql, total;
};

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Floats per pdg chunk record: C + 4, rounded up to a whole 128-byte line.
__host__ __device__ constexpr int pdg_stride(int C) { return (C + 4 + 31) / 32 * 32; }

static inline WsLayout ws_layout(int64_t NBH, int64_t NC, int C, int dirs, size_t mt_bytes, int64_t dv, bool plo) {
  WsLayout L;
  size_t off = 0;
  const size_t nch = (size_t)NBH * (size_t)NC;
  L.tri = off; off = align_up(off + nch * C * C * mt_bytes, 256);
  L.pqk = off; off = align_up(off + nch * C * C * mt_bytes, 256);
  L.sc = off;  off = align_up(off + (size_t)dirs * nch * C * 16, 256);
  L.pdg = off; off = align_up(off + (size_t)dirs * nch * pdg_stride(C) * 4, 256);
  L.rdy = off; off = align_up(off + nch * 4, 256);
  L.pfl = off; off = align_up(off + (dirs == 2 ? nch * (size_t)(dv / 16) * 4 : 0), 256);
  L.pql = off; off = align_up(off + (plo ? nch * C * C * 2 : 0), 256);
  L.total = off;
  return L;
}

// Arguments shared by both kernels.
struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const float* state_in;
  float* state_out;
  float* out;
  void* tri;
  void* pqk;
  float4* sc;
  float* pdg;
  unsigned* ready;     // rdy, above
  unsigned* part_flags;  // pfl, above (bidirectional bf16 scans; else null)
  void* pq_lo;           // pql, above (exclusive readouts on bf16 operands; else null)
  int64_t B, T, H, NC;
  int dv;
  int fwd_on, rev_on;  // which directions are computed
  int dirs;            // number of computed directions (slots)
  int zero_out;        // the preparation kernel fills `out` with the "not written yet" pattern (bidirectional fp32)
  int erase;           // 1: delta rule; 0: erase-free variant (no -beta k k^T term: L = 0, T = I)
  int excl_fwd, excl_rev;  // 1: that direction reads before the token's own write (no self term)
};

// Whether a preparation pass at chunk length C stores its workspace at
// agent scope (see bstore16_ws): beside the chain, or for a small pass; and
// always at 16 and 128 tokens, where plain stores measured slower on large
// passes too (480p bidirectional, 128-token chunks: 0.669 against 0.688 ms;
// 16-token chunks: 0.213 against 0.222 ms).
template <int C>
__device__ __forceinline__ bool ws_agent_stores(const ScanArgs& a) {
  constexpr int64_t kSmallPass = 2048;  // (chunk, sequence) items
  if constexpr (C == 16 || C == 128) return true;
  return a.ready != nullptr || a.NC * a.B * a.H < kSmallPass;
}

// Arguments of the frame-wise operator's kernels.  Workspace, per
// (direction slot, batch*head, frame): minv = (I + A_t)^{-1} [dk][dk], bmat =
// B_t [dv][dk], sfr = the state after the frame [dv][dk] (all fp32).
struct VdaArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;  // [dirs][B][NF][H], one per frame
  const float* beta;       // [dirs][B][T][H]
  const float* state_in;
  float* state_out;
  float* out;
  float* minv;
  float* bmat;
  float* sfr;
  int64_t B, T, H, NF, frame;
  int dv;
  int dirs, fwd_on, rev_on;
  int additive;             // 1: S_t = a S (I - A/U) + B / sqrt(U)
  int lag;                  // readout lag in frames
  const void* gate;         // epilogue gate logits, or null
  const float* norm_weight; // epilogue weights [dv]
  float norm_eps;
};

struct VdaLayout {
  size_t minv, bmat, sfr, total;
};

static inline VdaLayout vda_layout(int64_t NBH, int64_t NF, int dirs, int64_t dk, int64_t dv) {
  VdaLayout L;
  const size_t nfr = (size_t)dirs * (size_t)NBH * (size_t)NF;
  size_t off = 0;
  L.minv = off; off = align_up(off + nfr * dk * dk * 4, 256);
  L.bmat = off; off = align_up(off + nfr * dv * dk * 4, 256);
  L.sfr = off;  off = align_up(off + nfr * dv * dk * 4, 256);
  L.total = off;
  return L;
}

}  // namespace gdn

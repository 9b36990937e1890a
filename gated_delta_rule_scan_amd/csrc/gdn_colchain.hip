// State chain for bf16 operands: column-owning chain waves.
//
// The chunked scan (derivation in the preparation kernel) walks the chunks of
// one (batch, head, direction) in order; per chunk, with the entry state S
// (dv x dk, fp32),
//
//   Y = K S^T,   X = beta * (V - (e^g rk) * Y),   Vnew = X + strict(Tinv) X,
//   S' = e^{g_last} S + (e^{g_last - g} rk * Vnew)^T K,
//   O  = (e^g rq) * (Q S^T) + P Vnew          (P: decayed q^.k^ with the self terms),
//
// the chunk form of S_t = a_t S_{t-1}(I - b_t k^_t k^_t^T) + b_t v_t k^_t^T,
// o_t = S_t q^_t.
//
// Work split.  A workgroup owns a (batch, head, direction) sequence and
// 16*NT value columns.  Each of its NT chain waves owns 16 of those columns of
// the state over every dk, so Y, X, Vnew and the state update of its columns
// need nothing from another wave: every matrix-core result is, in registers,
// the operand of the next product.  Two index orders make that so:
//   * token order tau: row m of row tile rt of Y (and of X and Vnew) is token
//     32 (rt/2) + 8 (m/4) + 4 (rt%2) + m%4, so the four rows a lane holds in a
//     result tile are the four consecutive tokens the next product's operand
//     wants in that lane (the k and triangle rows are staged in this order);
//   * dk order pi: row m of state tile 2 ks + u is dk 32 ks + 8 (m/4) + 4 u +
//     m%4, so the state accumulators, rounded to bf16, are directly the
//     operand of Y = K S^T (the transposed k operand of the update is read in
//     this order).
// The chain's critical path is therefore register-only: Y (matrix cores, k
// from LDS) -> X (fp32) -> strict(Tinv) X (matrix cores) -> scaled Vnew as
// hi + lo bf16 parts -> state update (matrix cores, transposed k from LDS).
// Each of NT readout waves takes the chunk one step later: it reads the
// chunk's entry state and Vnew (hi + lo) that its chain wave left in LDS and
// computes the transposed output tile O^T = S Q^T + Vnew^T P^T, so each lane
// stores four consecutive values of one output row.  One barrier per step.
//
// Operand staging.  Every operand a wave reads from LDS arrives there by
// direct buffer-to-LDS loads (16 bytes per lane, 1 KB per instruction; the
// per-token records 4 bytes per lane), issued a step before its use into a
// two-slot ring per role by one more wave, the loader: the chain slot holds
// k (rows in tau order), the strict inverse triangle (rows in tau order),
// the value tile and the chunk scales; the readout slot holds q, the decayed
// q.k triangle and the chunk scales.  The compute waves issue no staging
// load, so none of them is held up while the address unit takes one.  Tiles
// are XOR-swizzled in 16-byte pieces so the operand reads are free of bank
// conflicts.  The loader waits for its own loads before each step's barrier
// (an explicit vmcnt, not a fence); the ring slots and the exchange buffers
// are distinct arrays, so the compiler can tell every LDS read from the
// loads in flight.
//
// Bidirectional scans run the two directions in separate workgroups (ids 8
// apart).  Chunk c is visited first by the direction that reaches it at the
// lower step index (the forward one for the first half of the chunks, the
// reverse one for the second half): that visitor stores its readout, the
// other adds it to its own.  A readout wave signals its stored partial
// through a flag per chunk and 16 columns (cleared by the preparation
// kernel, which has finished before the chain starts):
//   * the flag of visit v is stored at readout step v + 3, without a wait:
//     the barrier that ends step v + 2 already counted the stores of step
//     v + 1 out (each step issues its loads before its stores);
//   * a second visitor loads the flag two steps before its readout and the
//     partial one step before if the flag was set by then; otherwise it polls
//     the flag (bounded) and loads the partial at the readout;
//   * every readout wave, on reaching its first second visit, waits for its
//     own stores and publishes all its flags.  First visits precede second
//     visits in every workgroup, so no wave ever waits while holding an
//     unpublished flag, and neither direction can wait for the other in a
//     cycle.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4v;

namespace {

// s_waitcnt immediate (gfx9 encoding): vmcnt(n), lgkmcnt(0), expcnt at its maximum.
template <int n>
struct WaitVmLds {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  static constexpr int value = (n & 15) | ((n >> 4) << 14) | (7 << 4);
};

// The step barrier: this wave's own loads counted out (vmcnt(n)), its LDS
// writes done, then s_barrier.  The empty asm statements keep the compiler
// from moving memory accesses across it (a __syncthreads() would also make
// the compiler wait for every direct-to-LDS load in flight).
template <int n>
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(WaitVmLds<n>::value);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void mem_fence_compiler() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(rsrc_t r, lds_u8* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, 0, 0, 0);
}
// 4 bytes per lane into LDS at lds + 4 * lane.
__device__ __forceinline__ void dma4(rsrc_t r, lds_u8* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, (int)voff, 0, 0, 0);
}

__device__ __forceinline__ v4s tr16(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)const_cast<lds_u8*>(p));
}

// token order of the chain's product rows (see the file comment)
__host__ __device__ constexpr int tau(int rt, int m) { return 32 * (rt >> 1) + 8 * (m >> 2) + 4 * (rt & 1) + (m & 3); }

// PREC: 0, the readout's entry state and the decayed q.k tile in bf16; 1,
// the state as bf16 hi + lo parts (scans with the readout epilogue, whose
// per-row normalisation magnifies the error of small rows); 2, also the tile
// as hi + lo parts in the directions that read before the token's own write
// (exclusive readouts: outputs ten times smaller than the terms they sum).
template <int DK, int C, int NT, int PREC>
struct Col {
  static constexpr bool SLO = PREC >= 1, PLO = PREC >= 2;
  static constexpr int DT = 16 * NT;             // value columns per workgroup
  static constexpr int RT = C / 16;              // 16-token row tiles per chunk
  static constexpr int KC = C / 32;              // 32-token k-chunks
  static constexpr int KS = DK / 32;             // 32-wide dk slices
  static constexpr int SRT = DK / 16;            // 16-row dk tiles of the state
  static constexpr int KROWB = DK * 2;           // bytes per k / q row
  static constexpr int TROWB = C * 2;            // bytes per triangle row
  static constexpr int VROWB = DT * 2;           // bytes per value-tile row
  static constexpr int KB = C * KROWB, TB = C * TROWB, VB = C * VROWB;
  // chain slot: k | Tinv | v | scales | the head of the chunk record (its
  // decay; one 4-byte-per-lane load of 256 bytes)
  static constexpr int CK = 0, CT = CK + KB, CV = CT + TB, CS = CV + VB, CP = CS + 1024, CSLOT = CP + 256;
  // readout slot: q | P | [PLO: P's low parts in a direction reading before
  // the token's own write, else zeros] | e^g rq per token | the self-term
  // remainders per token (the last two: one 4-byte-per-lane load each)
  static constexpr int RQ = 0, RP = RQ + KB, RL = RP + TB;
  static constexpr int RS = RL + (PLO ? TB : 0), RD = RS + 256, RSLOT = RD + 256;
  // exchange, per chain wave: entry-state fragments (bf16; with SLO also
  // their low parts), Vnew (fp32, the eight values of a k-chunk operand
  // fragment per lane)
  static constexpr int XS = 0, XSL = KS * 1024, XV = XSL + (SLO ? KS * 1024 : 0), XJ = XV + KC * 2048,
                       XSLOT = NT * XJ;
  // loads per slot: 1 KB each, but the chain's last and the readout's last two (256 B)
  static constexpr int NDC = CP / 1024 + 1, NDR = RS / 1024 + 2;
  static_assert(KB % 1024 == 0 && TB % 1024 == 0 && VB % 1024 == 0, "whole 1-KB loads");
  static_assert(C == 32 || C == 64, "chunk");
};

// XOR swizzle of the 16-byte pieces of a k / q row and of a triangle row:
// the 16 rows one operand read touches land on distinct banks.
template <int DK>
__device__ __forceinline__ int swz_kq(int row) { return DK == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int C>
__device__ __forceinline__ int swz_t(int row) { return C == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3); }

// Where the tokens and pieces of one staged chunk come from.  Region kinds:
enum : int { R_KTAU = 0, R_QNAT = 1, R_TTAU = 2, R_PNAT = 3, R_VAL = 4, R_RAW = 5 };

template <int DK, int C, int NT>
__device__ __forceinline__ uint32_t dma_voff(int kind, int ii, int lane, uint32_t HDB, uint32_t HVB) {
  using L = Col<DK, C, NT, 0>;
  const int b = ii * 1024 + 16 * lane;  // byte within the staged region
  if (kind == R_KTAU || kind == R_QNAT) {
    const int rho = b / L::KROWB, q = (b % L::KROWB) >> 4;
    const int p = q ^ swz_kq<DK>(rho);
    const int t = kind == R_KTAU ? tau(rho >> 4, rho & 15) : rho;
    return (uint32_t)t * HDB + (uint32_t)p * 16u;
  }
  if (kind == R_TTAU || kind == R_PNAT) {
    const int rho = b / L::TROWB, q = (b % L::TROWB) >> 4;
    const int p = q ^ swz_t<C>(rho);
    const int r = kind == R_TTAU ? tau(rho >> 4, rho & 15) : rho;
    return (uint32_t)(r * L::TROWB + p * 16);
  }
  if (kind == R_VAL) {
    const int rho = b / L::VROWB, piece = (b % L::VROWB) >> 4;
    return (uint32_t)rho * HVB + (uint32_t)piece * 16u;
  }
  return (uint32_t)b;
}

constexpr int kColPollLimit = 1 << 23;      // about a second of re-reads
constexpr int kColReadyPollLimit = 1 << 23;

__device__ __forceinline__ f32x4 col_load_fresh(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 17);
  f32x4 f;
  __builtin_memcpy(&f, &v, 16);
  return f;
}

__device__ __forceinline__ uint32_t col_flag_fresh(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 17);
}

__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (bf16)a[i];
    r[4 + i] = (bf16)b[i];
  }
  return r;
}

// hi + lo bf16 parts of eight fp32 values (hi = rounded value, lo = rounded remainder)
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (bf16)a[i];
    hi[4 + i] = (bf16)b[i];
    lo[i] = (bf16)(a[i] - (float)hi[i]);
    lo[4 + i] = (bf16)(b[i] - (float)hi[4 + i]);
  }
}

__device__ __forceinline__ bf16x8 lds_frag(const lds_u8* p) { return *(const lds_bf16x8*)p; }
__device__ __forceinline__ void lds_put(lds_u8* p, bf16x8 v) { *(lds_bf16x8*)p = v; }
__device__ __forceinline__ float lds_f(const lds_u8* p) { return *(const lds_f32*)p; }
__device__ __forceinline__ f32x4 lds_f4(const lds_u8* p) { return *(const lds_f32x4v*)p; }

__device__ __forceinline__ bf16x8 and_mask(bf16x8 f, const uint32_t (&m)[4]) {
  uint32_t w[4];
  __builtin_memcpy(w, &f, 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] &= m[i];
  __builtin_memcpy(&f, w, 16);
  return f;
}

// 8-element keep mask of a fragment lane: element e is column col0 + e of row `row`
__device__ __forceinline__ void make_mask(uint32_t (&m)[4], int row, int col0, bool upper, bool diag) {
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int col = col0 + e;
    const bool keep = (upper ? (col > row) : (col < row)) || (diag && col == row);
    if (keep) m[e / 2] |= 0xffffu << (16 * (e % 2));
  }
}

}  // namespace

template <int DK, int C, int NT, bool BI, int PREC>
__global__ __launch_bounds__(128 * NT + 64) void column_chain_kernel(ScanArgs a, int rev_single, int ntiles, int nbh) {
  using L = Col<DK, C, NT, PREC>;
  constexpr bool SLO = L::SLO, PLO = L::PLO;
  using M = Mma<bf16>;
  constexpr int RT = L::RT, KC = L::KC, KS = L::KS, SRT = L::SRT, DT = L::DT;

  __shared__ __align__(1024) unsigned char cs0_[L::CSLOT], cs1_[L::CSLOT];  // chain ring
  __shared__ __align__(1024) unsigned char rs0_[L::RSLOT], rs1_[L::RSLOT];  // readout ring
  __shared__ __align__(1024) unsigned char xs0_[L::XSLOT], xs1_[L::XSLOT];  // exchange, by step parity
  __shared__ __align__(256) unsigned char pf_[256];                          // L2-prefetch sink, never read
  lds_u8* const cs0 = (lds_u8*)cs0_;
  lds_u8* const cs1 = (lds_u8*)cs1_;
  lds_u8* const rs0 = (lds_u8*)rs0_;
  lds_u8* const rs1 = (lds_u8*)rs1_;
  lds_u8* const xs0 = (lds_u8*)xs0_;
  lds_u8* const xs1 = (lds_u8*)xs1_;
  lds_u8* const pfs = (lds_u8*)pf_;

  // workgroup id -> (sequence, value tile, direction): the value tiles of one
  // (batch, head) share an XCD; the two directions of a tile are 8 ids apart
  const int ndir = BI ? 2 : 1;
  const int id = blockIdx.x;
  const int xcd = id & 7, kk = id >> 3;
  const int chain = (kk / (ntiles * ndir)) * 8 + xcd;
  const int dslot = BI ? (kk & 1) : 0;
  const int tile = (kk / ndir) % ntiles;
  if (chain >= nbh) return;
  const int NC = (int)a.NC;
  const int64_t T = a.T, H = a.H;
  const int64_t b = chain / H, h = chain % H;
  const int dv = a.dv;
  const int dv0 = tile * DT;
  const bool rev = BI ? (dslot == 1) : (rev_single != 0);
  const int slot = dslot;
  // this direction reads before the token's own write and adds P's low parts
  const bool plo_dir = PLO && (rev ? a.excl_rev : a.excl_fwd);

  const int lane = threadIdx.x & 63;
  // Roles by hardware wave: wave 0 is the loader, then the chain and the
  // readout waves.  A workgroup's waves are dealt to the four SIMDs in order,
  // so with two chain and two readout waves the fifth wave shares a SIMD with
  // wave 0: that way a readout wave shares with the loader and each chain wave
  // has a SIMD of its own (measured on MI355X: 480p bidirectional chain 2%
  // faster than with the loader beside a chain wave).
  const int w = (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) + 2 * NT) % (2 * NT + 1);
  const bool chain_wave = w < NT;
  const bool loader = w == 2 * NT;  // the staging wave
  const int j = w % NT;             // 16-column sub-tile of a chain or readout wave
  const int l16 = lane & 15, g4 = lane >> 4;

  const uint32_t HDB = (uint32_t)(H * DK * 2);  // token pitch of q, k (bytes)
  const uint32_t HVB = (uint32_t)(H * dv * 2);  // token pitch of v
  const uint32_t HOB = (uint32_t)(H * dv * 4);  // token pitch of out
  const size_t nch = (size_t)a.B * a.H * NC;
  const char* kbase = static_cast<const char*>(a.k) + (size_t)((b * T * H + h) * DK) * 2;
  const char* qbase = static_cast<const char*>(a.q) + (size_t)((b * T * H + h) * DK) * 2;
  const char* vbase = static_cast<const char*>(a.v) + (size_t)((b * T * H + h) * dv + dv0) * 2;
  char* obase = reinterpret_cast<char*>(a.out) + (size_t)((b * T * H + h) * dv + dv0) * 4;
  const char* trib = static_cast<const char*>(a.tri) + (size_t)chain * NC * L::TB;
  const char* pqkb = static_cast<const char*>(a.pqk) + (size_t)chain * NC * L::TB;
  const char* pqlb = PLO && a.pq_lo ? static_cast<const char*>(a.pq_lo) + (size_t)chain * NC * L::TB : pqkb;
  const char* scb = reinterpret_cast<const char*>(a.sc) + ((size_t)slot * nch + (size_t)chain * NC) * C * 16;
  const char* pdb = reinterpret_cast<const char*>(a.pdg) + ((size_t)slot * nch + (size_t)chain * NC) * pdg_stride(C) * 4;
  const rsrc_t rnone = make_rsrc(obase, 0u);

  auto chunk_at = [&](int s) { return rev ? NC - 1 - s : s; };
  // Slot order of a chunk's row tiles: slot pair p holds the two 16-token
  // tiles of k-chunk kd_of(p), the k-chunks in reverse order for the reverse
  // direction.  In slot order both directions' triangles are lower, so which
  // k-chunks a slot's products take is known at compile time; only LDS
  // addresses depend on the direction.
  auto kd_of = [&](int p) { return rev ? KC - 1 - p : p; };
  auto rt_of = [&](int u) { return 2 * kd_of(u >> 1) + (u & 1); };
  auto first_visit = [&](int s) {  // bidirectional: this workgroup visits chunk_at(s) first
    const int so = NC - 1 - s;
    return !BI || s < so || (s == so && !rev);
  };

  const size_t sbase = (((size_t)slot * a.B + b) * a.H + h) * (size_t)dv * DK;

  if (chain_wave) {
    // ======================= chain wave =======================
    // state accumulators: tile srt = 2 ks + u, lane (l16, g4) element i holds
    // S[dv0 + 16 j + l16][32 ks + 8 g4 + 4 u + i]
    f32x4 Sacc[SRT];
    const int col = dv0 + 16 * j + l16;
#pragma unroll
    for (int srt = 0; srt < SRT; ++srt) {
      const int ks = srt >> 1, u = srt & 1;
      Sacc[srt] = a.state_in ? *reinterpret_cast<const f32x4*>(a.state_in + sbase + (size_t)col * DK + 32 * ks + 8 * g4 + 4 * u)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // triangle masks of the diagonal k-chunk of each row tile (strict)
    uint32_t tmask[RT][4];
#pragma unroll
    for (int u = 0; u < RT; ++u) make_mask(tmask[u], tau(rt_of(u), l16), 32 * kd_of(u >> 1) + 8 * g4, rev, false);

    // one chain step on chunk chunk_at(s), held by `cur`
    auto chain_step = [&](const lds_u8* cur, lds_u8* xw, int s) {
      const lds_u8* Kt = cur + L::CK;
      const lds_u8* Tt = cur + L::CT;
      const lds_u8* Vt = cur + L::CV;
      const lds_u8* Sc = cur + L::CS;
      const lds_u8* Pd = cur + L::CP;
      lds_u8* X = xw + j * L::XJ;
      // k fragments of Y, read first (they are in LDS since the last step)
      bf16x8 ka[RT][KS];
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        const int rho = 16 * rt_of(u) + l16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[u][ks] = lds_frag(Kt + rho * L::KROWB + (((4 * ks + g4) ^ swz_kq<DK>(rho)) << 4));
      }

      // entry state as bf16 operand fragments (dk 32 ks + 8 g4 .. + 7 of column l16)
      bf16x8 sb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (SLO) {
          bf16x8 sl;
          split8(Sacc[2 * ks], Sacc[2 * ks + 1], sb[ks], sl);
          lds_put(X + L::XSL + ks * 1024 + lane * 16, sl);
        } else {
          sb[ks] = pack8(Sacc[2 * ks], Sacc[2 * ks + 1]);
        }
        lds_put(X + L::XS + ks * 1024 + lane * 16, sb[ks]);
      }
      // Y = K S^T (rows in token order tau, row tiles in slot order); the row
      // tiles are independent accumulators, so each slice's products issue
      // back to back
      f32x4 y[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) y[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) y[rt] = M::mma(ka[rt][ks], sb[ks], y[rt]);
      }
      // X = beta (V - e^g rk Y); lane (l16, g4) of slot u holds tokens t0 .. t0 + 3
      f32x4 x[RT], dsc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int t0 = 32 * kd_of(rt >> 1) + 8 * g4 + 4 * (rt & 1);
        const v4s t4 = tr16(Vt + (t0 + (l16 >> 2)) * L::VROWB + (16 * j + 4 * (l16 & 3)) * 2);
        bf16x4 v4;
        __builtin_memcpy(&v4, &t4, 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 s4 = lds_f4(Sc + (t0 + i) * 16);  // {beta, e^g rk, e^g rq, e^(gn-g) rk}
          x[rt][i] = s4[0] * ((float)v4[i] - s4[1] * y[rt][i]);
          dsc[rt][i] = s4[3];
        }
      }
      // Vnew = X + strict(Tinv) X (X exact in fp32; the strict part on bf16 operands)
      bf16x8 xb[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) xb[kc] = pack8(x[2 * kc], x[2 * kc + 1]);
      f32x4 vn[RT];
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        f32x4 acc = x[u];
        const int rho = 16 * rt_of(u) + l16;
        const int p = u >> 1;  // slot pair of the diagonal
#pragma unroll
        for (int m = 0; m <= p; ++m) {  // the k-chunks of this direction's triangle
          bf16x8 ta = lds_frag(Tt + rho * L::TROWB + (((4 * kd_of(m) + g4) ^ swz_t<C>(rho)) << 4));
          if (m == p) ta = and_mask(ta, tmask[u]);
          acc = M::mma(ta, xb[m], acc);
        }
        vn[u] = acc;
      }
      // Vnew (fp32) for the readout; the scaled Vs (hi + lo) for the update
      bf16x8 vsh[KC], vsl[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        *(lds_f32x4v*)(X + L::XV + kc * 2048 + lane * 32) = vn[2 * kc];
        *(lds_f32x4v*)(X + L::XV + kc * 2048 + lane * 32 + 16) = vn[2 * kc + 1];
        split8(vn[2 * kc] * dsc[2 * kc], vn[2 * kc + 1] * dsc[2 * kc + 1], vsh[kc], vsl[kc]);
      }
      // S = e^{g_last} S + K^T Vs: the transposed k fragment of state tile
      // srt = 2 ks + u and k-chunk kc holds k[32 kc + 8 g4 + e][pi(srt, l16)]
      const float gn = lds_f(Pd);  // the record's head
#pragma unroll
      for (int srt = 0; srt < SRT; ++srt) Sacc[srt] = Sacc[srt] * gn;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
        for (int srt = 0; srt < SRT; ++srt) {
          const int ks = srt >> 1, u = srt & 1;
          bf16x8 kt;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int rho = 16 * (2 * kd_of(kc) + hh) + 4 * g4 + (l16 >> 2);  // row of token 32 kd + 8 g4 + 4 hh + l16 / 4
            const int p = 4 * ks + (l16 & 3);
            const v4s r = tr16(Kt + rho * L::KROWB + ((p ^ swz_kq<DK>(rho)) << 4) + 8 * u);
            __builtin_memcpy(reinterpret_cast<char*>(&kt) + 8 * hh, &r, 8);
          }
          Sacc[srt] = M::mma(kt, vsh[kc], Sacc[srt]);
          Sacc[srt] = M::mma(kt, vsl[kc], Sacc[srt]);
        }
      }
    };

    if (NC > 0) {
      step_barrier<0>();  // the loader's prologue: chunk 0 staged
      int s = 0;
      for (; s + 1 < NC; s += 2) {
        chain_step(cs0, xs0, s);
        step_barrier<0>();
        chain_step(cs1, xs1, s + 1);
        step_barrier<0>();
      }
      if (s < NC) {
        chain_step(cs0, xs0, s);
        step_barrier<0>();
        ++s;
      }
      // the readout's last step
      step_barrier<0>();
    }
    // final state
    if (a.state_out) {
#pragma unroll
      for (int srt = 0; srt < SRT; ++srt) {
        const int ks = srt >> 1, u = srt & 1;
        *reinterpret_cast<f32x4*>(a.state_out + sbase + (size_t)col * DK + 32 * ks + 8 * g4 + 4 * u) = Sacc[srt];
      }
    }
  } else if (!loader) {
    // ======================= readout wave =======================
    // P masks of the diagonal k-chunk of each 16-token output tile, in slot
    // order (the self terms kept unless this direction reads before the
    // token's own write)
    const bool self = !(rev ? a.excl_rev : a.excl_fwd);
    const uint32_t plk = plo_dir ? ~0u : 0u;  // P's low parts: read in this direction
    uint32_t pmask[RT][4], dmask[RT][4];  // dmask: the element of this lane's own token (none: all zero)
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int tt = rt_of(u);
      make_mask(pmask[u], 16 * tt + l16, 32 * kd_of(u >> 1) + 8 * g4, rev, self);
      const int e0 = 16 * tt + l16 - (32 * kd_of(u >> 1) + 8 * g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) dmask[u][i] = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (self && e == e0) dmask[u][e / 2] |= 0xffffu << (16 * (e % 2));
    }
    const rsrc_t ro = make_rsrc(obase, (uint32_t)(T - 1) * HOB + DT * 4);
    const uint32_t out_lane = (uint32_t)(16 * j + 4 * g4) * 4u;
    auto out_off = [&](int c, int tt) { return (uint32_t)(c * C + 16 * tt + l16) * HOB + out_lane; };
    bool pq_gave_up = false;

    // ---- bidirectional combine flags (see the file comment) ----
    const int nfl = dv >> 4;          // flag columns per chunk
    const int fcol = (dv0 >> 4) + j;  // this wave's
    const rsrc_t rfl = BI && a.part_flags ? make_rsrc(a.part_flags + (size_t)chain * NC * nfl, (uint32_t)(NC * nfl) * 4u)
                                          : rnone;
    auto flag_off = [&](int v) { return (uint32_t)(chunk_at(min(v, NC - 1)) * nfl + fcol) * 4u; };
    const int nfirst = BI ? (rev ? NC / 2 : (NC + 1) / 2) : NC;  // first visits are 0 .. nfirst - 1
    int pub_next = 0;  // first visits before this one have their flags stored
    // the flag of visit v, if it is an unpublished first visit (else a store
    // through the empty resource: one store either way); every lane stores
    // the same word
    auto publish = [&](int v) {
      const bool now = v >= pub_next && v < nfirst;
      bstore4u_agent(now ? rfl : rnone, flag_off(v < 0 ? 0 : v), 1u);
      if (now) pub_next = v + 1;
    };
    // the flag of visit v (a second visit), for the partial load a step later
    auto load_flag = [&](uint32_t& fl, int v) {
      if constexpr (BI) fl = col_flag_fresh(v < NC && !first_visit(v) ? rfl : rnone, flag_off(v));
    };
    // the partial of visit v, if its flag was set when loaded (`got`; else
    // zeros: the readout polls)
    auto load_partial = [&](f32x4 (&pq)[RT], bool got, int v) {
      if constexpr (BI) {
        const rsrc_t rp = got ? ro : rnone;
        const int c = chunk_at(min(v, NC - 1));
#pragma unroll
        for (int u = 0; u < RT; ++u) pq[u] = col_load_fresh(rp, out_off(c, rt_of(u)));
      }
    };

    // Readout step s: load the flag of visit s + 1 and the partial of visit
    // s, then read out visit s - 1 from slot `cur` (staged by the loader in
    // step s - 1) and exchange `xr`.  Every step issues the same vector
    // memory operations in the same order -- a flag store, the flag, the
    // partial, the output stores -- through an empty resource where there is
    // nothing to load or store.
    // The step-end waits count on that, and so do the waits the compiler
    // derives for the loop from every path into it.
    auto read_step = [&](const lds_u8* cur, const lds_u8* xr, f32x4 (&pq)[RT], bool got,
                         f32x4 (&pq_next)[RT], bool& got_next, uint32_t fl_s, uint32_t& fl_next, int s) {
      // whether visit s's partial is published (its flag was loaded a step
      // ago; tested first, while only the last step's tail is in flight)
      if constexpr (BI) got_next = s < NC && !first_visit(s) && __builtin_amdgcn_readfirstlane(fl_s) != 0u;
      if constexpr (BI) {
        if (s - 1 == nfirst && nfirst > 0) {
          // the first second visit: every flag of this wave stored first
          __builtin_amdgcn_s_waitcnt(kWaitVmem);
          while (pub_next < nfirst) publish(pub_next);
        }
        publish(s - 3);  // its stores were counted out by the barrier ending step s - 1
      }
      mem_fence_compiler();
      load_flag(fl_next, s + 1);
      load_partial(pq_next, got_next, s);
      mem_fence_compiler();
      if (s == 0) {
        // no readout yet: the output stores go to the empty resource
#pragma unroll
        for (int tt = 0; tt < RT; ++tt) bstore16(rnone, out_off(0, tt), f32x4{0.f, 0.f, 0.f, 0.f});
        return;
      }
      const int sp = s - 1;
      const int c = chunk_at(sp);
      const lds_u8* Qt = cur + L::RQ;
      const lds_u8* Pt = cur + L::RP;
      const lds_u8* Sc = cur + L::RS;
      const lds_u8* Pd = cur + L::RD;
      const lds_u8* X = xr + j * L::XJ;
      const bool add = BI && !first_visit(sp);
      if (BI && add && !got) {
        // the partial was not published two steps ago: wait for its flag
        bool ok = false;
        if (!pq_gave_up) {
          int n = 0;
          for (; n < kColPollLimit; ++n) {
            if (__builtin_amdgcn_readfirstlane(col_flag_fresh(rfl, flag_off(sp))) != 0u) break;
            __builtin_amdgcn_s_sleep(2);
          }
          ok = n < kColPollLimit;
          pq_gave_up = !ok;
        }
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int u = 0; u < RT; ++u) pq[u] = ok ? col_load_fresh(ro, out_off(c, rt_of(u))) : f32x4{nan, nan, nan, nan};
        // waited for here, so that the compiler does not make the common
        // path wait as if these loads were in flight there
        __builtin_amdgcn_s_waitcnt(kWaitVmem);
      }
      bf16x8 sr[KS], vh[KC], vl[KC];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sr[ks] = lds_frag(X + L::XS + ks * 1024 + lane * 16);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const f32x4 v0 = *(const lds_f32x4v*)(X + L::XV + kc * 2048 + lane * 32);
        const f32x4 v1 = *(const lds_f32x4v*)(X + L::XV + kc * 2048 + lane * 32 + 16);
        split8(v0, v1, vh[kc], vl[kc]);
      }
      // The slots' products are independent (one accumulator each) and take
      // k-chunks known at compile time: every fragment is read first, then
      // the products run slice by slice across the slots, so each product's
      // accumulator was written RT products earlier.
      bf16x8 qf[RT][KS];
      float zs[RT], rmd[RT];
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        const int t = 16 * rt_of(u) + l16;  // this lane's token
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[u][ks] = lds_frag(Qt + t * L::KROWB + (((4 * ks + g4) ^ swz_kq<DK>(t)) << 4));
        zs[u] = lds_f(Sc + t * 4);  // e^g rq of the token
        rmd[u] = lds_f(Pd + t * 4);  // the self term's remainder
      }
      // Z^T = S Q^T
      f32x4 o[RT];
#pragma unroll
      for (int u = 0; u < RT; ++u) o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 sl;
        if constexpr (SLO) sl = lds_frag(X + L::XSL + ks * 1024 + lane * 16);  // the state's low parts
#pragma unroll
        for (int u = 0; u < RT; ++u) {
          o[u] = M::mma(sr[ks], qf[u][ks], o[u]);
          if constexpr (SLO) o[u] = M::mma(sl, qf[u][ks], o[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < RT; ++u) o[u] = o[u] * zs[u];
      // + Vnew^T P^T over the k-chunks of each slot's triangle: chunk m
      // enters the slots of pairs p >= m (the diagonal one, p == m, masked)
#pragma unroll
      for (int m = 0; m < KC; ++m) {
        bf16x8 pf[RT], pl[RT];
#pragma unroll
        for (int u = 2 * m; u < RT; ++u) {
          const int t = 16 * rt_of(u) + l16;
          const int poff = t * L::TROWB + (((4 * kd_of(m) + g4) ^ swz_t<C>(t)) << 4);
          pf[u] = lds_frag(Pt + poff);
          if ((u >> 1) == m) pf[u] = and_mask(pf[u], pmask[u]);
          if constexpr (PLO) {
            // P's low part (with Vnew's hi part: the product's next order),
            // zero in a direction that reads its token's own write
            uint32_t lm[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) lm[i] = ((u >> 1) == m ? pmask[u][i] : ~0u) & plk;
            pl[u] = and_mask(lds_frag(cur + L::RL + poff), lm);
          }
        }
#pragma unroll
        for (int u = 2 * m; u < RT; ++u) o[u] = M::mma(vh[m], pf[u], o[u]);
#pragma unroll
        for (int u = 2 * m; u < RT; ++u) o[u] = M::mma(vl[m], pf[u], o[u]);
        if constexpr (PLO) {
#pragma unroll
          for (int u = 2 * m; u < RT; ++u) o[u] = M::mma(vh[m], pl[u], o[u]);
        }
        // the self terms' remainders (P holds them rounded): a diagonal
        // product with Vnew's hi part in the slots of pair m
#pragma unroll
        for (int u = 2 * m; u < 2 * m + 2; ++u) {
          const bf16 r = (bf16)rmd[u];
          bf16x8 dg;
#pragma unroll
          for (int e = 0; e < 8; ++e) dg[e] = r;
          o[u] = M::mma(vh[m], and_mask(dg, dmask[u]), o[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        const uint32_t off = out_off(c, rt_of(u));
        if constexpr (BI) {
          // the partial is zero on a first visit, which stores its readout
          // for the other direction (agent scope: the other direction loads
          // it); a second visit's sum is read by no later step of this
          // launch, so it takes a plain store, which completes sooner and so
          // holds up less the waits of the wave's later loads (memory
          // operations complete in issue order; measured: bidir720 chain
          // 3.35 -> 3.24 ms)
          if (add) bstore16(ro, off, o[u] + pq[u]);
          else bstore16_agent(ro, off, o[u] + pq[u]);
        } else {
          bstore16(ro, off, o[u]);
        }
      }
    };

    f32x4 pqa[RT], pqb[RT];
#pragma unroll
    for (int tt = 0; tt < RT; ++tt) pqa[tt] = pqb[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool ga = false, gb = false;
    uint32_t fa = 0u, fb = 0u;
    // memory operations a readout wave leaves in flight at a step's end: the
    // flag and the partials it loads ahead (bidirectional) and its output
    // stores
    constexpr int kTail = BI ? 2 * RT + 1 : RT;
    if (NC > 0) {
      step_barrier<0>();  // the loader's prologue
      load_flag(fa, 0);
      // step 0 loads the partial of visit 0; no readout yet
      read_step(rs1, xs1, pqb, gb, pqa, ga, fa, fb, 0);
      step_barrier<kTail>();
      // then steps 1 .. NC: odd steps read slot 0, even steps slot 1
      int s = 1;
      for (; s + 1 <= NC; s += 2) {
        read_step(rs0, xs0, pqa, ga, pqb, gb, fb, fa, s);
        step_barrier<kTail>();
        read_step(rs1, xs1, pqb, gb, pqa, ga, fa, fb, s + 1);
        step_barrier<kTail>();
      }
      if (s <= NC) {
        read_step(rs0, xs0, pqa, ga, pqb, gb, fb, fa, s);
        step_barrier<kTail>();
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmem);
      if constexpr (BI) {
        // flags not yet stored (short sequences)
        while (pub_next < nfirst) publish(pub_next);
      }
    }
  } else {
    // ======================= loader wave =======================
    // Every operand load of the workgroup: at step s the chain slot of chunk
    // s + 1 and the readout slot of chunk s (direct buffer-to-LDS loads, all
    // 1-KB units of both slots), the L2 prefetch three chunks ahead and, with
    // the preparation running concurrently, the chunk-ready flags.  A
    // buffer-to-LDS load holds up the wave that issues it until the compute
    // unit's address unit takes it; issued by the chain and readout waves,
    // these loads delayed their products (measured at the 480p bidirectional
    // shape: ~1,400 of ~5,400 cycles per step before the first product).
    uint32_t voffc[L::NDC], voffr[L::NDR];
#pragma unroll
    for (int i = 0; i < L::NDC; ++i) {
      const int byte = i * 1024;
      voffc[i] = byte < L::CT   ? dma_voff<DK, C, NT>(R_KTAU, (byte - L::CK) / 1024, lane, HDB, HVB)
                 : byte < L::CV ? dma_voff<DK, C, NT>(R_TTAU, (byte - L::CT) / 1024, lane, HDB, HVB)
                 : byte < L::CS ? dma_voff<DK, C, NT>(R_VAL, (byte - L::CV) / 1024, lane, HDB, HVB)
                 : byte < L::CP ? 16u * lane
                                : 4u * lane;  // the record's head (the chunk decay)
    }
#pragma unroll
    for (int i = 0; i < L::NDR; ++i) {
      const int byte = i * 1024;
      if (i < L::RS / 1024) {
        voffr[i] = byte < L::RP   ? dma_voff<DK, C, NT>(R_QNAT, (byte - L::RQ) / 1024, lane, HDB, HVB)
                   : byte < L::RL ? dma_voff<DK, C, NT>(R_PNAT, (byte - L::RP) / 1024, lane, HDB, HVB)
                   : plo_dir      ? dma_voff<DK, C, NT>(R_PNAT, (byte - L::RL) / 1024, lane, HDB, HVB)
                                  : 16u * lane;
      } else {
        // e^g rq: the third float of each token's scale record; the
        // remainders: the record after its 16-byte head
        voffr[i] = i == L::RS / 1024 ? 16u * lane + 8u : 16u + 4u * lane;
      }
    }
    auto rows_of = [&](int c) { return (uint32_t)(T - (int64_t)c * C); };  // valid tokens from the chunk start (>= 1)
    auto stage_chain = [&](lds_u8* slotp, int c) {
      const uint32_t rows = rows_of(c);
      const rsrc_t rkq = make_rsrc(kbase + (size_t)c * C * HDB, (rows - 1) * HDB + DK * 2);
      const rsrc_t rtp = make_rsrc(trib + (size_t)c * L::TB, (uint32_t)L::TB);
      const rsrc_t rsc = make_rsrc(scb + (size_t)c * C * 16, (uint32_t)(C * 16));
      const rsrc_t rpd = make_rsrc(pdb + (size_t)c * pdg_stride(C) * 4, (uint32_t)((C + 4) * 4));
      const rsrc_t rv = make_rsrc(vbase + (size_t)c * C * HVB, (rows - 1) * HVB + DT * 2);
#pragma unroll
      for (int i = 0; i < L::NDC; ++i) {
        const int byte = i * 1024;
        if (byte >= L::CP) {
          dma4(rpd, slotp + byte, voffc[i]);
        } else {
          const rsrc_t r = byte < L::CT ? rkq : byte < L::CV ? rtp : byte < L::CS ? rv : rsc;
          dma16(r, slotp + byte, voffc[i]);
        }
      }
    };
    auto stage_read = [&](lds_u8* slotp, int c) {
      const uint32_t rows = rows_of(c);
      const rsrc_t rkq = make_rsrc(qbase + (size_t)c * C * HDB, (rows - 1) * HDB + DK * 2);
      const rsrc_t rtp = make_rsrc(pqkb + (size_t)c * L::TB, (uint32_t)L::TB);
      const rsrc_t rsc = make_rsrc(scb + (size_t)c * C * 16, (uint32_t)(C * 16));
      const rsrc_t rpd = make_rsrc(pdb + (size_t)c * pdg_stride(C) * 4, (uint32_t)((C + 4) * 4));
      // PLO: the low parts of P, or loads through the empty resource (the
      // same count either way)
      const rsrc_t rpl = make_rsrc(pqlb + (size_t)c * L::TB, (uint32_t)L::TB);
#pragma unroll
      for (int i = 0; i < L::NDR; ++i) {
        const int byte = i * 1024;
        if (i < L::RS / 1024) {
          const rsrc_t r = byte < L::RP ? rkq : byte < L::RL ? rtp : plo_dir ? rpl : rnone;
          dma16(r, slotp + byte, voffr[i]);
        } else if (i == L::RS / 1024) {
          dma4(rsc, slotp + L::RS, voffr[i]);
        } else {
          dma4(rpd, slotp + L::RD, voffr[i]);
        }
      }
    };

    // ---- L2 prefetch of the tiles the value-tile workgroups of one
    // sequence share (k and Tinv, q and P) ----
    // Those workgroups run in step and ask for the same lines at the same
    // time, so every one of them would wait for the same HBM fill.  Instead
    // the loaders of a sequence's tiles each touch every ntiles-th 128-byte
    // line of the chunk three ahead, one line per lane, with 4-byte loads
    // into a sink nobody reads: when the chunk is staged two steps later,
    // its lines are in this XCD's L2.  (Measured at the 480p bidirectional
    // shape: state chain 1.20 -> 1.09 ms with the prefetch; two, five or
    // eight chunks ahead, or also the unshared value tile: slower.)  With the
    // preparation running concurrently (a.ready set) a chunk's prepared
    // tiles are prefetched only once its ready flag, loaded a step before,
    // has read ready: a prepared tile read before its flag could leave a
    // stale line in this XCD's L2 (the preparation workgroup may run on
    // another XCD), which the staging load would hit.  (Measured at the 720p
    // causal shape: chain 1.80 ms beside the preparation with only k and q
    // prefetched, 1.59 ms with the prepared tiles too.)
    constexpr int LPR = L::KROWB / 128;  // 128-byte lines per k (q) row
    constexpr int KL = L::KB / 128, TL = L::TB / 128;
    static_assert(KL <= 128 && TL <= 64, "a workgroup's lines fit one lane each when ntiles >= 2");
    const bool pf_prepared = a.ready == nullptr;  // prepared tiles are final before the chain starts
    const int lk = tile + ntiles * lane;  // this lane's line of the k (q) tile and of a triangle
    const uint32_t pfk = lk < KL ? (uint32_t)((lk / LPR) * HDB + (lk % LPR) * 128) : 0xFFFFFFF0u;
    const uint32_t pft = lk < TL ? (uint32_t)(lk * 128) : 0xFFFFFFF0u;
    auto prefetch = [&](int c, bool prepared) {
      const uint32_t rows = rows_of(c);
      const rsrc_t rk = make_rsrc(kbase + (size_t)c * C * HDB, (rows - 1) * HDB + DK * 2);
      const rsrc_t rq = make_rsrc(qbase + (size_t)c * C * HDB, (rows - 1) * HDB + DK * 2);
      const bool pp = pf_prepared || prepared;
      const rsrc_t rt = pp ? make_rsrc(trib + (size_t)c * L::TB, (uint32_t)L::TB) : rnone;
      const rsrc_t rp = pp ? make_rsrc(pqkb + (size_t)c * L::TB, (uint32_t)L::TB) : rnone;
      dma4(rk, pfs, pfk);
      dma4(rt, pfs, pft);
      dma4(rq, pfs, pfk);
      dma4(rp, pfs, pft);
    };

    // ready flags of the concurrent preparation (0 = ready; without a.ready
    // they read 0 through an empty resource).  A wait that expires (a
    // preparation pass starved of the GPU) returns true once; later waits are
    // skipped.
    const rsrc_t rrdy = a.ready ? make_rsrc(a.ready + (size_t)chain * NC, (uint32_t)NC * 4u) : rnone;
    bool gave_up = false;
    auto ensure_ready = [&](uint32_t fl, int c) {
      bool expired = false;
      if (__builtin_amdgcn_readfirstlane(fl) != 0u && !gave_up) {
        int n = 0;
        for (; n < kColReadyPollLimit; ++n) {
          __builtin_amdgcn_s_sleep(2);
          if (__builtin_amdgcn_readfirstlane(col_flag_fresh(rrdy, (uint32_t)c * 4u)) == 0u) break;
        }
        expired = gave_up = n == kColReadyPollLimit;
      }
      return expired;
    };
    // The chunk whose wait expired: its staged scales and decay become NaN
    // (after its loads have landed), so X, Vnew and the state the chain
    // waves compute from it are NaN, and with them every later output and
    // the final state -- never values computed from a stale workspace.
    auto poison = [&](lds_u8* slotp) {
      __builtin_amdgcn_s_waitcnt(kWaitVmem);
      const float nan = __builtin_nanf("");
      *(lds_f32x4v*)(slotp + L::CS + 16 * lane) = f32x4{nan, nan, nan, nan};
      *(lds_f32*)(slotp + L::CP + 4 * lane) = nan;
    };
    auto flag_of = [&](int s) { return col_flag_fresh(rrdy, (uint32_t)chunk_at(min(s, NC - 1)) * 4u); };

    // One loader step: the same loads in the same order at every step (the
    // last steps restage the last chunk into idle slots), which the step-end
    // waits and the compiler's loop waits count on.  `fl` is chunk s + 1's
    // ready flag, loaded two steps ago, and receives chunk s + 3's; `gu` is
    // chunk s + 3's, loaded a step ago (it gates that chunk's prepared-tile
    // prefetch), and `gn` receives chunk s + 4's.
    constexpr int kLTail = 6;  // loads left in flight at a step's end: the four prefetch loads and two flags
    auto load_step = [&](lds_u8* cnext, lds_u8* rcur, uint32_t& fl, uint32_t gu, uint32_t& gn, int s) {
      const int cn = chunk_at(min(s + 1, NC - 1));
      const bool expired = ensure_ready(fl, cn);
      mem_fence_compiler();
      stage_chain(cnext, cn);
      if (expired) poison(cnext);
      mem_fence_compiler();
      stage_read(rcur, chunk_at(min(s, NC - 1)));
      mem_fence_compiler();
      prefetch(chunk_at(min(s + 3, NC - 1)), __builtin_amdgcn_readfirstlane(gu) == 0u);
      mem_fence_compiler();
      fl = flag_of(s + 3);
      gn = flag_of(s + 4);
      mem_fence_compiler();
    };
    if (NC > 0) {
      const bool expired = ensure_ready(flag_of(0), chunk_at(0));
      // after the first flag, a step's loads in a step's order (the readout
      // slot staged here is read in no step)
      uint32_t fa = flag_of(1);
      mem_fence_compiler();
      stage_chain(cs0, chunk_at(0));
      if (expired) poison(cs0);
      mem_fence_compiler();
      stage_read(rs1, chunk_at(0));
      mem_fence_compiler();
      prefetch(chunk_at(min(1, NC - 1)), false);
      mem_fence_compiler();
      uint32_t fb = flag_of(2), ga = flag_of(3), gb = 0u;
      mem_fence_compiler();
      step_barrier<kLTail>();  // chunk 0 in the chain slot
      // steps 0 .. NC: the chain slot of chunk s + 1 and the readout slot of chunk s
      int s = 0;
      for (; s + 1 <= NC; s += 2) {
        load_step(cs1, rs0, fa, ga, gb, s);
        step_barrier<kLTail>();
        load_step(cs0, rs1, fb, gb, ga, s + 1);
        step_barrier<kLTail>();
      }
      if (s <= NC) {
        load_step(cs1, rs0, fa, ga, gb, s);
        step_barrier<kLTail>();
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmem);  // the last restages and prefetch
    }
  }
}

template <int DK, int C, int NT, bool BI, int PREC>
hipError_t launch_column_chain(const ScanArgs& a, int rev_single, hipStream_t stream, hipFuncAttributes* query) {
  if (query) return hipFuncGetAttributes(query, reinterpret_cast<const void*>(&column_chain_kernel<DK, C, NT, BI, PREC>));
  const int ntiles = a.dv / (16 * NT);
  const int nbh = (int)(a.B * a.H);
  const unsigned nblocks = (unsigned)chain_blocks(nbh, a.dv, NT, BI ? 2 : 1);
  hipLaunchKernelGGL((column_chain_kernel<DK, C, NT, BI, PREC>), dim3(nblocks), dim3(128 * NT + 64), 0, stream, a,
                     rev_single, ntiles, nbh);
  return hipGetLastError();
}

#define GDN_INST_COL(DK, C, NT, BI, PREC) \
  template hipError_t launch_column_chain<DK, C, NT, BI, PREC>(const ScanArgs&, int, hipStream_t, hipFuncAttributes*);
// PREC 2 (exclusive readouts): 16-column tiles only (its LDS would not fit 32)
#define GDN_INST_COL_P(DK, C, NT, BI) GDN_INST_COL(DK, C, NT, BI, 0) GDN_INST_COL(DK, C, NT, BI, 1) \
  GDN_INST_COL_IF_NT1(DK, C, NT, BI)
#define GDN_INST_COL_IF_NT1(DK, C, NT, BI) GDN_INST_COL_PLO_##NT(DK, C, BI)
#define GDN_INST_COL_PLO_1(DK, C, BI) GDN_INST_COL(DK, C, 1, BI, 2)
#define GDN_INST_COL_PLO_2(DK, C, BI)
#define GDN_INST_COL_D(DK, C, NT) GDN_INST_COL_P(DK, C, NT, false) GDN_INST_COL_P(DK, C, NT, true)
#define GDN_INST_COL_N(DK, C) GDN_INST_COL_D(DK, C, 1) GDN_INST_COL_D(DK, C, 2)
GDN_INST_COL_N(64, 32)
GDN_INST_COL_N(64, 64)
GDN_INST_COL_N(128, 32)
GDN_INST_COL_N(128, 64)

}  // namespace gdn

// State-chain kernel: the sequential part of the chunked gated delta-rule
// scan, with the chunk outputs fused in.
//
// One workgroup owns a (batch, head, value tile) -- `16*NT` rows of the fp32
// state S (dv x dk) -- and walks the chunks in scan order.  With the chunk
// quantities from the preparation kernel (Tinv, decayed Q^K^^T, scales) and the
// raw q, k, v of the chunk, one step is
//
//   Y = K S^T,  Z = Q S^T                    (matrix cores; K, Q raw)
//   X = beta * (V - (e^g rk) * Y)            (fp32, pseudo-values vs. entry state)
//   Vnew = X + strict(Tinv) X                (matrix cores; X kept exact in fp32)
//   O = (e^g rq) * Z + P Vnew                (P: decayed q^.k^, self terms on the diagonal)
//   S = e^{g_last} S + (e^{g_last-g} rk * Vnew)^T K    (matrix cores, fp32 accumulate)
//
// which is the chunked form of S_t = a_t S_{t-1}(I - b_t k^_t k^_t^T) +
// b_t v_t k^_t^T, o_t = S_t q^_t (derivation in the preparation kernel).
//
// Bidirectional scans ("Video DeltaNet", "Methodology in Plain English": a
// forward and a backward recurrent state whose readouts are added) run the
// two directions in separate workgroups, which the hardware overlaps freely
// (two direction groups on one workgroup barrier would make every wave wait
// for the slowest of both at every phase, and per-group LDS barriers are
// slow under the groups' LDS traffic).  Every chunk is visited by both: the
// forward workgroup visits chunk s at its step s, the reverse one at its step
// NC-1-s.  The first visitor (the forward one for the first half of the
// chunks, the reverse one for the second half) stores its readout; the
// second loads that partial a step ahead, adds its own readout and stores the
// sum.  The preparation kernel fills `out` with an all-ones NaN pattern that
// no readout produces, so the second visitor knows when the partial has
// arrived: while any of its elements still holds the pattern, it re-reads
// them past its L1 cache (rare: only near the middle of the sequence do the
// two visits come close in time).  The first visits of a workgroup come
// before all of its second visits, so a first visitor never waits; partner
// workgroups have nearby ids, and with in-order dispatch every waiting
// workgroup's partner runs, so every wait ends (the polls are bounded too).

// Every global access goes through a raw buffer resource whose extent is the
// valid part of the workgroup's whole chain (built once; a chunk is a 32-bit
// byte offset): reads past it return zero and writes past it are dropped.
// Rows past the end of the sequence therefore need no clamping and no
// branches, and an access that must not happen this step (the partial of a
// first visit, the store of a step that has nothing to store) goes through a
// resource with an empty extent.  All loads of a step are issued by every wave
// of a role unconditionally, a step ahead of their use, so no prefetch ever
// forces a wait on the in-order memory counter.
//
// A workgroup has two roles of four waves each, on the same four SIMDs.  The
// chain waves carry the state: Y, X, Vnew and the state update, the critical
// path.  The readout waves compute Z and the chunk outputs beside them, so
// those leave the critical path; the two roles meet at the step's three
// barriers (phases below).
//
// Workgroups are numbered so that all value tiles of one (batch, head) land
// on the same XCD (consecutive workgroups are dealt round-robin over the
// eight XCDs), so the tiles share the chunk operands through one L2.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

// Tokens a chunk's products contract over: the chunk itself, padded to one
// 32-wide matrix-core contraction for 16-token chunks (the padding entries
// are zero in every operand, so the products are those of the 16 tokens).
template <int C>
struct ChainK {
  static constexpr int CK = C < 32 ? 32 : C;
  static constexpr int KCN = CK / 32;  // 32-token contraction slices per chunk
};

template <typename MT, int DK, int C, int NT>
struct ChainSmem {
  static constexpr int ES = (int)sizeof(MT);
  static constexpr int EP = 16 / ES;
  static constexpr int CK = ChainK<C>::CK;
  static constexpr int TP = CK + EP;  // pitch of token-contiguous rows
  static constexpr int SP = DK + EP;  // pitch of the state copy
  static constexpr int DT = 16 * NT;
  // k tile of the chunk.  bf16: row-major [C][DK + 8] (the transposed
  // operand of the state update is read with transposing LDS reads).  The
  // pitch is 68 dwords: the 16-byte row stores are then free of bank
  // conflicts on gfx950 (a 72-dword pitch doubles their cost; measured), and
  // the transposing reads cost the same at either pitch.
  // fp32: token-contiguous [DK][TP].
  static constexpr bool KROW = ES == 2;
  static constexpr int KP = DK + 8;
  static constexpr int k_elems = KROW ? CK * KP : DK * TP;
  // bf16 operands: Vnew and the scaled update vectors are carried as hi + lo
  // bf16 pairs (two products each), so their rounding stays at fp32 level.
  static constexpr bool SPLIT = ES == 2;
  static constexpr int NVT = SPLIT ? 5 : 3;  // token-contiguous value arrays
  static constexpr int per_group = k_elems + NVT * DT * TP + DT * SP;  // elements
  // Staged per-chunk operands shared by a direction group (bytes): the
  // per-token scales, the self-term remainders with the chunk decay, the
  // value tile.  Double buffered by step parity.
  static constexpr int ST_SC = 0;
  static constexpr int ST_PD = C * 16;
  static constexpr int ST_GN = ST_PD;  // the record starts with the chunk's decay
  static constexpr int ST_V = ST_PD + (C + 4) * 4;
  static constexpr int ST_BYTES = ST_V + C * DT * ES;
};

template <typename MT, int DT, int C>
struct VTile {
  static constexpr int LPR = DT * (int)sizeof(MT) / 16;  // 16-byte pieces per token row
  static constexpr int NVI = (C * LPR + 127) / 128;      // loads per wave (two waves share the tile)
};

// Raw operands of one chunk, loaded a step ahead of their use, per role.
// Chain waves: the k rows of their token tile and the matching rows of the
// strict inverse triangle (matrix-core fragments), 16 bytes per lane of the
// group-shared operands (wave 0: scales, wave 1: self-term remainders and
// chunk decay, waves 2-3: the value tile), which go to LDS at the end of the
// step, and the ready flag of the chunk the stage is loaded with next (read
// two steps ahead; 0 = ready).
template <typename MT, int DK, int C, int NT>
struct StageC {
  typedef typename Mma<MT>::frag frag;
  static constexpr int RPW = C > 64 ? C / 64 : 1;  // token row tiles per wave
  frag kf[RPW][DK / 32];
  frag tf[RPW][ChainK<C>::KCN];
  f32x4 cv[VTile<MT, 16 * NT, C>::NVI];
  uint32_t rdy;
};
// Readout waves: the q rows of their token tile, the matching rows of the
// decayed q^.k^ triangle, and for a bidirectional second visit the other
// direction's readout of the chunk (per output tile of the wave).
template <typename MT, int DK, int C, int NT>
struct StageR {
  typedef typename Mma<MT>::frag frag;
  static constexpr int RPW = C > 64 ? C / 64 : 1;
  frag qf[RPW][DK / 32];
  frag pf[RPW][ChainK<C>::KCN];
  f32x4 pq[(C / 16 * NT + 3) / 4];
};

__device__ __forceinline__ bool tri_needed(bool rev, int kc, int rt) {
  // k-chunks (32 tokens) of a 16-row tile that hold strictly-lower (forward)
  // or strictly-upper (reverse) entries
  return rev ? (32 * kc + 31 > 16 * rt) : (32 * kc <= 16 * rt + 15);
}

// Bit masks that keep the lower (forward) or upper (reverse) elements of a
// triangle fragment, with or without the diagonal; only the k-chunk that
// contains the diagonal needs one (the others keep everything), and they are
// loop-invariant per lane.
template <typename MT>
struct FragMask {
  static constexpr int NW = (int)(sizeof(typename Mma<MT>::frag) / 4);
  uint32_t m[NW];
  // `limit`: columns from it on lie past the chunk (16-token chunks, whose
  // fragments span 32 columns) and are dropped
  __device__ __forceinline__ void make(int row, int col0, bool upper, bool diag, bool active, int limit) {
#pragma unroll
    for (int i = 0; i < NW; ++i) m[i] = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = col0 + e;
      const bool keep = col < limit && (!active || (upper ? (col > row) : (col < row)) || (diag && col == row));
      if (keep) {
        if (sizeof(MT) == 2) m[e / 2] |= 0xffffu << (16 * (e % 2));
        else m[e] = 0xffffffffu;
      }
    }
  }
  __device__ __forceinline__ typename Mma<MT>::frag apply(typename Mma<MT>::frag f) const {
    uint32_t w[NW];
    __builtin_memcpy(w, &f, sizeof(f));
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] &= m[i];
    __builtin_memcpy(&f, w, sizeof(f));
    return f;
  }
};

// hi + lo bf16 split of four fp32 values (hi = rounded value, lo = rounded
// remainder), written as two 8-byte LDS stores.
__device__ __forceinline__ void store_split4(bf16* hi_p, bf16* lo_p, f32x4 x) {
  bf16x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = (bf16)x[i];
    l[i] = (bf16)(x[i] - (float)h[i]);
  }
  *reinterpret_cast<bf16x4*>(hi_p) = h;
  *reinterpret_cast<bf16x4*>(lo_p) = l;
}


// All-ones NaN: the value the preparation kernel fills `out` with before a
// bidirectional scan, meaning "not written yet".  First visitors store their
// readouts with canonical NaNs (an input NaN's payload could otherwise carry
// the pattern through the arithmetic), so they never produce it.
constexpr uint32_t kUnwritten = 0xFFFFFFFFu;

__device__ __forceinline__ bool any_unwritten(f32x4 p) {
  return __float_as_uint(p[0]) == kUnwritten || __float_as_uint(p[1]) == kUnwritten ||
         __float_as_uint(p[2]) == kUnwritten || __float_as_uint(p[3]) == kUnwritten;
}

// 16-byte load that misses the L1 cache (system-scope cache policy), for
// re-reading data another compute unit writes.
__device__ __forceinline__ f32x4 bload16_fresh(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 17);
  f32x4 f;
  __builtin_memcpy(&f, &v, 16);
  return f;
}

// Bound on the re-reads of one partial (about a second at ~0.14 us per
// re-read, measured on MI355X).  Partners are dispatched together, so a wait
// is normally short; a partner can start late only when other work holds
// compute units.  A workgroup that ever exhausts the bound stops waiting for
// the rest of the launch, so a launch always ends; the outputs it then adds
// to an unwritten partial keep the fill pattern (a NaN), so they cannot pass
// unnoticed.
constexpr int kPollLimit = 1 << 23;

// 4-byte flag load that misses the L1 cache, as a uint32
__device__ __forceinline__ uint32_t bload4_fresh(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 17);
}

// Bound on the polls for one chunk's ready flag (about a second at ~0.14 us
// per poll, measured on MI355X: far longer than any preparation pass that
// fits in device memory takes, also when it queues behind another call's pass
// on the shared library stream); a
// workgroup that ever exhausts it stops waiting for the rest of the launch,
// so a launch always ends, and sets its state and pseudo-values to NaN: every later
// output of its chain and its final state are then NaN (the canonical quiet
// NaN, never the "not written yet" pattern), so a starved preparation pass
// cannot pass unnoticed.
constexpr int kReadyPollLimit = 1 << 23;

// Waves per state-chain workgroup: four chain waves (one per SIMD), which
// carry the state, and four readout waves beside them, which compute Z = Q S^T
// and the chunk outputs (measured on MI355X: the chain 2% faster than with
// the readout on the chain waves, bitwise the same results).  (Eight waves
// splitting the chain's own work, one output tile each, measured 1.4x slower:
// every wave then reads the whole update operand from LDS.)
template <int C, int NT>
struct ChainWaves {
  static constexpr int value = 8;
};

template <typename MT, int DK, int C, int NT, bool BI>
__global__ __launch_bounds__((64 * ChainWaves<C, NT>::value)) void chain_kernel(ScanArgs a, int rev_single, int ntiles,
                                                                              int nbh) {
  using M = Mma<MT>;
  using frag = typename M::frag;
  using SM = ChainSmem<MT, DK, C, NT>;
  constexpr int ES = SM::ES;
  constexpr int TP = SM::TP, SP = SM::SP, DT = SM::DT;
  using VT = VTile<MT, DT, C>;
  constexpr int RT = C / 16;              // token row tiles per chunk
  constexpr int KCN = ChainK<C>::KCN;     // 32-token contraction slices per chunk
  constexpr int NWC = 4;                        // chain waves; readout waves follow them
  constexpr int RPW = RT > NWC ? RT / NWC : 1;  // token row tiles per wave (wave wr: tiles wr + NWC r)
  constexpr int UPW = (RT * NT + NWC - 1) / NWC;  // chunk-output tiles per wave
  constexpr int SRT = DK / 16;                    // state row tiles (dk)
  constexpr int SUPW = SRT * NT / NWC;            // state tiles per chain wave
  constexpr bool SPLIT = SM::SPLIT;
  constexpr bool ALL_UNITS = (RT * NT) % NWC == 0;
  static_assert(ChainWaves<C, NT>::value == 2 * NWC, "one readout wave per chain wave");
  static_assert(SRT % NWC == 0 || NWC % SRT == 0, "state tiles split evenly over the waves");
  static_assert(NWC % RT == 0 || RT % NWC == 0, "every wave keeps the same number of token row tiles");
  static_assert(RPW == StageC<MT, DK, C, NT>::RPW && RPW == StageR<MT, DK, C, NT>::RPW, "stage layout");

  __shared__ __align__(16) MT smem[SM::per_group];
  __shared__ __align__(16) unsigned char stg[2][SM::ST_BYTES];

  // XCD-aware numbering: workgroup id -> (chain, value tile, direction); all
  // workgroups of one (batch, head) land on the same XCD, and the two
  // directions of a tile have ids 8 apart
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

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int cw = w & 3;  // chain wave's part of the group-shared loads (0: scales, 1: remainders, 2-3: value tile)
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wr = w & (NWC - 1);  // place among the chain waves (readout wave w mirrors chain wave w - NWC)
  const bool reader = w >= NWC;  // readout waves: Z = Q S^T and the chunk outputs
  // row tile of output unit j (u = wr + NWC j): tile wr % RT + NWC rj(j)
  auto rj = [](int j) { return RT > NWC ? j % RPW : 0; };

  constexpr bool KROW = SM::KROW;
  constexpr int KP = SM::KP;
  MT* KT = smem;                             // k tile (layout: see ChainSmem)
  MT* XT = KT + SM::k_elems;                 // [DT][TP]  pseudo-values X^T
  MT* VnT = XT + DT * TP;                    // [DT][TP]  Vnew^T (hi part)
  MT* VsT = VnT + DT * TP;                   // [DT][TP]  (scaled Vnew)^T (hi part)
  MT* VnL = VsT + DT * TP;                   // [DT][TP]  lo parts (bf16 operands only)
  MT* VsL = SPLIT ? VnL + DT * TP : VnL;
  MT* Sb = VsT + (SM::NVT - 2) * DT * TP;    // [DT][SP]  state copy (operand type)

  // ---- loop-invariant addressing: per-lane byte offsets within a chunk,
  // wave-uniform chunk bases and strides ----
  const uint32_t HDB = (uint32_t)(H * DK * ES);  // token pitch of q, k
  const uint32_t HVB = (uint32_t)(H * dv * ES);  // token pitch of v
  const uint32_t HOB = (uint32_t)(H * dv * 4);   // token pitch of out
  const size_t nch = (size_t)a.B * a.H * NC;
  const char* kbase = static_cast<const char*>(a.k) + (size_t)((b * T * H + h) * DK) * ES;
  const char* qbase = static_cast<const char*>(a.q) + (size_t)((b * T * H + h) * DK) * ES;
  const char* vbase = static_cast<const char*>(a.v) + (size_t)((b * T * H + h) * dv + dv0) * ES;
  char* obase = reinterpret_cast<char*>(a.out) + (size_t)((b * T * H + h) * dv + dv0) * 4;
  const char* trib = static_cast<const char*>(a.tri) + (size_t)chain * NC * C * C * ES;
  const char* pqkb = static_cast<const char*>(a.pqk) + (size_t)chain * NC * C * C * ES;
  int kq_row[RPW], o_row0[RPW];
  uint32_t kq_off[RPW], tri_off[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int rt = wr % RT + NWC * r;
    kq_row[r] = 16 * rt + l16;
    kq_off[r] = kq_row[r] * HDB + 8 * g4 * ES;
    tri_off[r] = (kq_row[r] * C + 8 * g4) * ES;
    o_row0[r] = 16 * rt + 4 * g4;
  }
  // triangle fragments: the k-chunks of this row tile that hold no element
  // of this direction's triangle are read past the buffer extent (zeros, see
  // the resources below); the diagonal k-chunk is masked (Tinv strictly, P
  // with its diagonal -- the self terms -- unless this direction reads
  // before the token's own write, which is exactly P without its diagonal)
  const bool self = !(rev ? a.excl_rev : a.excl_fwd);
  FragMask<MT> tmask[RPW][KCN], pmask[RPW][KCN];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int kc = 0; kc < KCN; ++kc) {
      const int kcd = (wr % RT + NWC * r) / 2;  // k-chunk holding the row tile's diagonal
      tmask[r][kc].make(kq_row[r], 32 * kc + 8 * g4, rev, false, kc == kcd, C);
      pmask[r][kc].make(kq_row[r], 32 * kc + 8 * g4, rev, self, kc == kcd, C);
    }
  // readout offset of unit column tile 0 (transposed tile: token kq_row, four
  // columns from 4 g4)
  uint32_t out_off[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) out_off[r] = kq_row[r] * HOB + 16 * g4;
  // bf16 operands: the self term's remainder enters as a diagonal fragment;
  // in k-chunk kc this lane (row kq_row of P) holds element `kq_row - 32 kc -
  // 8 g4` of it when that lies in 0..7 (only ever in the k-chunk of the diagonal)
  FragMask<MT> diag_only[RPW][KCN];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int kc = 0; kc < KCN; ++kc) {
#pragma unroll
      for (int i = 0; i < FragMask<MT>::NW; ++i) diag_only[r][kc].m[i] = 0u;
      const int e0 = self ? kq_row[r] - 32 * kc - 8 * g4 : -1;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e == e0) {
          if (sizeof(MT) == 2) diag_only[r][kc].m[e / 2] |= 0xffffu << (16 * (e % 2));
          else diag_only[r][kc].m[e] = 0xffffffffu;
        }
    }
  // group-shared operand loads: which source this wave reads, per-lane offsets
  // and where each piece lands in the staging buffer
  const char* cbase;
  uint32_t cstride;  // bytes per chunk
  uint32_t cbytes;   // extent of the whole chain
  uint32_t c_off[VT::NVI], c_lds[VT::NVI];
  if (cw == 0) {
    cbase = reinterpret_cast<const char*>(a.sc) + ((size_t)slot * nch + (size_t)chain * NC) * C * 16;
    cstride = C * 16;
    cbytes = (uint32_t)NC * cstride;
  } else if (cw == 1) {
    cbase = reinterpret_cast<const char*>(a.pdg) + ((size_t)slot * nch + (size_t)chain * NC) * pdg_stride(C) * 4;
    cstride = pdg_stride(C) * 4;
    cbytes = (uint32_t)NC * cstride;
  } else {
    cbase = vbase;
    cstride = C * HVB;
    cbytes = (uint32_t)(T - 1) * HVB + DT * ES;
  }
#pragma unroll
  for (int n = 0; n < VT::NVI; ++n) {
    if (cw == 0) {
      const int idx = (lane + 64 * n) % C;
      c_off[n] = idx * 16;
      c_lds[n] = SM::ST_SC + idx * 16;
    } else if (cw == 1) {
      const int idx = min(lane, C / 4);
      c_off[n] = idx * 16;
      c_lds[n] = SM::ST_PD + idx * 16;
    } else {
      const int idx = min((cw - 2) * 64 + n * 128 + lane, C * VT::LPR - 1);
      const int row = idx / VT::LPR, part = idx % VT::LPR;
      c_off[n] = row * HVB + part * 16;
      c_lds[n] = SM::ST_V + idx * 16;
    }
  }

  // ---- whole-chain resources, built once: an access adds its chunk's byte
  // offset (32 bits; the host bounds every extent below 4 GiB) to its
  // per-lane offset.  Token rows past the end of the sequence lie past the
  // extent (loads read zero, stores are dropped); an access that must not
  // happen this step goes through `rnone` (empty extent) ----
  const rsrc_t rnone = make_rsrc(obase, 0u);
  const uint32_t kq_ext = (uint32_t)(T - 1) * HDB + DK * ES;
  const rsrc_t rk = make_rsrc(kbase, kq_ext), rq = make_rsrc(qbase, kq_ext);
  const rsrc_t rc = make_rsrc(cbase, cbytes);
  const rsrc_t ro = make_rsrc(obase, (uint32_t)(T - 1) * HOB + DT * 4);
  const uint32_t tri_bytes = (uint32_t)NC * (C * C * ES);
  rsrc_t rtk[RPW][KCN], rpk[RPW][KCN];  // triangle k-chunks a row tile never needs: zeros
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int kc = 0; kc < KCN; ++kc) {
      const bool need = tri_needed(rev, kc, wr % RT + NWC * r);
      rtk[r][kc] = make_rsrc(trib, need ? tri_bytes : 0u);
      rpk[r][kc] = make_rsrc(pqkb, need ? tri_bytes : 0u);
    }
  // the chunks' ready flags, when the preparation kernel runs concurrently
  // (a.ready set; 0 = ready): a chunk's prepared operands are read only once
  // its flag is 0.  Without a.ready the flags read as 0 (empty extent).
  const rsrc_t rrdy = a.ready ? make_rsrc(a.ready + (size_t)chain * NC, (uint32_t)NC * 4u) : rnone;
  bool rdy_gave_up = false;
  auto ensure_ready = [&](uint32_t fl, int c) {
    // first test outside any loop: a loop that reloads the tested value makes
    // the compiler wait for every load in flight at its head
    if (__builtin_amdgcn_readfirstlane(fl) != 0u && !rdy_gave_up) {
      int n = 0;
      for (; n < kReadyPollLimit; ++n) {
        __builtin_amdgcn_s_sleep(2);
        if (__builtin_amdgcn_readfirstlane(bload4_fresh(rrdy, (uint32_t)c * 4u)) == 0u) break;
      }
      rdy_gave_up = n == kReadyPollLimit;
    }
  };
  auto ready_flag = [&](int c) { return bload4_fresh(rrdy, (uint32_t)c * 4u); };
  auto kq_at = [&](int c) { return (uint32_t)c * (C * HDB); };
  auto out_at = [&](int c) { return (uint32_t)c * (C * HOB); };

  // ---- loaders (issued a step ahead) ----
  auto load_rows = [&](frag (*dst)[DK / 32], const rsrc_t rs, int c) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint32_t o = kq_off[r] + kq_at(c);
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) dst[r][ks] = bload_frag<MT>(rs, o + 32 * ks * ES);
    }
  };
  auto load_coop = [&](auto& f, int c) {
    const uint32_t o = (uint32_t)c * cstride;
#pragma unroll
    for (int n = 0; n < VT::NVI; ++n) f.cv[n] = bload16(rc, c_off[n] + o);
  };
  auto load_tf = [&](auto& f, int c) {  // chain waves
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint32_t o = tri_off[r] + (uint32_t)c * (C * C * ES);
#pragma unroll
      for (int kc = 0; kc < KCN; ++kc) f.tf[r][kc] = bload_frag<MT>(rtk[r][kc], o + 32 * kc * ES);
    }
  };
  auto load_pf = [&](auto& f, int c) {  // readout waves
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint32_t o = tri_off[r] + (uint32_t)c * (C * C * ES);
#pragma unroll
      for (int kc = 0; kc < KCN; ++kc) f.pf[r][kc] = bload_frag<MT>(rpk[r][kc], o + 32 * kc * ES);
    }
  };
  auto stash = [&](const auto& f, int buf) {  // group-shared pieces of a loaded stage -> LDS
#pragma unroll
    for (int n = 0; n < VT::NVI; ++n) *reinterpret_cast<f32x4*>(&stg[buf][c_lds[n]]) = f.cv[n];
  };

  // 16-token chunks: the padding tokens of every token-contiguous operand
  // (the k tile's rows or columns 16..31, the value arrays' columns) stay
  // zero for the whole launch; the steps write only the chunk's own tokens
  if constexpr (C < 32) {
    for (int i = threadIdx.x; i < SM::per_group; i += 64 * ChainWaves<C, NT>::value) smem[i] = (MT)0.f;
    __syncthreads();
  }

  // ---- initial state into accumulators (S^T tiles) and the operand copy ----
  f32x4 Sacc[SUPW];
  const size_t sbase = (((size_t)slot * a.B + b) * a.H + h) * (size_t)dv * DK;
#pragma unroll
  for (int j = 0; j < SUPW; ++j) {
    const int u = wr + NWC * j;
    const int srt = u % SRT, sct = u / SRT;
    const size_t off = sbase + (size_t)(dv0 + 16 * sct + l16) * DK + 16 * srt + 4 * g4;
    Sacc[j] = a.state_in && !reader ? *reinterpret_cast<const f32x4*>(a.state_in + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (!reader) M::store4(Sb + (16 * sct + l16) * SP + 16 * srt + 4 * g4, Sacc[j][0], Sacc[j][1], Sacc[j][2], Sacc[j][3]);
  }

  auto chunk_at = [&](int s) { return rev ? NC - 1 - s : s; };
  // bidirectional: whether this workgroup visits chunk_at(s) before the other
  // direction does (see the file comment)
  auto first_visit = [&](int s) {
    const int so = NC - 1 - s;  // step at which the other direction visits the same chunk
    return !BI || s < so || (s == so && !rev);
  };

  // Readout of step sp (chunk chunk_at(sp)) by the readout waves, in the
  // step's last phase: O = (e^g rq) Z + P Vnew.  Everything it reads is
  // intact there: Z (registers, from the step's first phase), the P fragments
  // (the wave's own stage), Vnew (LDS until the next step's second phase) and
  // the staged scales (until the next step's last phase).  `on` = false:
  // nothing is stored.  Second visits of a bidirectional scan add the partial
  // the other direction stored (the stage's pq, loaded a step ahead and
  // checked just before).
  f32x4 Zp[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) Zp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto readout = [&](const auto& sp, const int s_prev, const bool on) {
    const unsigned char* sg = stg[s_prev & 1];
    frag pdiag[RPW];  // this lane's self-term remainder in every element (bf16 operands)
    if constexpr (SPLIT) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const bf16 x = (bf16)(*reinterpret_cast<const float*>(sg + SM::ST_PD + 16 + kq_row[r] * 4));
#pragma unroll
        for (int e = 0; e < 8; ++e) pdiag[r][e] = x;
      }
    }
    const int c = chunk_at(s_prev);
    const rsrc_t rs = on ? ro : rnone;
    float zs[RPW];  // e^g rq of the token
#pragma unroll
    for (int r = 0; r < RPW; ++r) zs[r] = *reinterpret_cast<const float*>(sg + SM::ST_SC + kq_row[r] * 16 + 8);
    const bool add = BI && !first_visit(s_prev);
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = wr + NWC * j;
      if (ALL_UNITS || u < RT * NT) {
        const int ct = u / RT, r = rj(j);
        f32x4 acc = Zp[j] * zs[r];
#pragma unroll
        for (int kc = 0; kc < KCN; ++kc) {
          const frag pf = pmask[r][kc].apply(sp.pf[r][kc]);
          const int o = (16 * ct + l16) * TP + 32 * kc + 8 * g4;
          const frag vh = M::load(VnT + o);
          acc = M::mma(vh, pf, acc);
          if constexpr (SPLIT) {
            acc = M::mma(M::load(VnL + o), pf, acc);
            // self-term remainder (pqk holds the rounded self term): a
            // diagonal product with the hi part of Vnew
            acc = M::mma(vh, diag_only[r][kc].apply(pdiag[r]), acc);
          }
        }
        if (add) acc += sp.pq[j];
        else if (BI) acc = canonical_nans(acc);  // a first visit: never the fill pattern
        // a first visit's readout is the other direction's partial: agent
        // scope, visible to it on any XCD once stored; sums and single-direction
        // readouts are read by no later step of this launch
        if (BI && !add) bstore16_agent(rs, out_off[r] + out_at(c) + ct * 64, acc);
        else bstore16(rs, out_off[r] + out_at(c) + ct * 64, acc);
      }
    }
  };

  // One step (chunk c = chunk_at(s); nx is loaded with chunk cn for the
  // next step), one lambda per role with the same three barriers.  Chain
  // waves (w < NWC) carry the state; readout waves compute Z = Q S^T and the
  // chunk outputs beside them, on the same SIMDs, so the chain waves'
  // critical path holds only Y, X, Vnew and the state update.
  //   phase A  chain: k tile -> LDS, Y = K S^T, X -> LDS
  //            readout: Z = Q S^T (the state copy is stable until phase C)
  //   phase B  chain: Vnew = X + strict(T) X -> LDS
  //            readout: next P fragments and partial (after phase A's wait on
  //            the ready flag of chunk cn)
  //   phase C  chain: state update, state copy and next scales -> LDS
  //            readout: O = (e^g rq) Z + P Vnew (Vnew intact until the next phase B)
  using FC = StageC<MT, DK, C, NT>;
  using FR = StageR<MT, DK, C, NT>;
  auto step_chain = [&](FC& st, FC& nx, const int s, const int cn) {
    const int buf = s & 1;
    const unsigned char* sg = stg[buf];
    f32x4 X[UPW];
    float4 sc[RPW][4];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[r][i] = *reinterpret_cast<const float4*>(sg + SM::ST_SC + (o_row0[r] + i) * 16);

    // [A] k tile into LDS; Y = K S^T; X
    if (wr < RT) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if constexpr (KROW) {
#pragma unroll
          for (int ks = 0; ks < DK / 32; ++ks)
            *reinterpret_cast<frag*>(KT + kq_row[r] * KP + 32 * ks + 8 * g4) = st.kf[r][ks];
        } else {
#pragma unroll
          for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) KT[(32 * ks + 8 * g4 + e) * TP + kq_row[r]] = (MT)M::get(st.kf[r][ks], e);
        }
      }
    }
    ensure_ready(nx.rdy, cn);  // before any read of chunk cn's prepared operands
    const bool poison = rdy_gave_up;  // see kReadyPollLimit
    if (poison) {
#pragma unroll
      for (int j = 0; j < SUPW; ++j) Sacc[j] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
    load_coop(nx, cn);
    load_rows(nx.kf, rk, cn);
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = wr + NWC * j;
      if (ALL_UNITS || u < RT * NT) {
        const int ct = u / RT, r = rj(j);
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
          y = M::mma(st.kf[r][ks], M::load(Sb + (16 * ct + l16) * SP + 32 * ks + 8 * g4), y);
        // raw values v[o_row0 + i][16 ct + l16], i = 0..3
        f32x4 vv;
        if constexpr (KROW) {
          const v4s t4 = lds_read_tr16(sg + SM::ST_V + ((o_row0[r] + (l16 >> 2)) * DT + 16 * ct + 4 * (l16 & 3)) * 2);
          bf16x4 b4;
          __builtin_memcpy(&b4, &t4, 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) vv[i] = (float)b4[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vv[i] = *reinterpret_cast<const float*>(sg + SM::ST_V + ((o_row0[r] + i) * DT + 16 * ct + l16) * 4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) X[j][i] = sc[r][i].x * (vv[i] - sc[r][i].y * y[i]);
        if (poison) X[j] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        M::store4(XT + (16 * ct + l16) * TP + o_row0[r], X[j][0], X[j][1], X[j][2], X[j][3]);
      }
    }
    __syncthreads();

    // [B] Vnew = X + strict(Tinv) X, and its scaled copy for the state update
    nx.rdy = ready_flag(chunk_at(min(s + 3, NC - 1)));  // what nx is loaded with two steps on
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = wr + NWC * j;
      if (ALL_UNITS || u < RT * NT) {
        const int ct = u / RT, r = rj(j);
        f32x4 acc = X[j];
#pragma unroll
        for (int kc = 0; kc < KCN; ++kc)
          acc = M::mma(tmask[r][kc].apply(st.tf[r][kc]), M::load(XT + (16 * ct + l16) * TP + 32 * kc + 8 * g4), acc);
        const int o = (16 * ct + l16) * TP + o_row0[r];
        f32x4 vs;
#pragma unroll
        for (int i = 0; i < 4; ++i) vs[i] = sc[r][i].w * acc[i];
        if constexpr (SPLIT) {
          store_split4(VnT + o, VnL + o, acc);
          store_split4(VsT + o, VsL + o, vs);
        } else {
          M::store4(VnT + o, acc[0], acc[1], acc[2], acc[3]);
          M::store4(VsT + o, vs[0], vs[1], vs[2], vs[3]);
        }
      }
    }
    __syncthreads();

    // [C] state update S^T = gn S^T + K^T Vs.  Chain wave wr owns the state
    // tiles u = wr + NWC j, i.e. dk tiles srt(js) and dv tiles sct(jt) below;
    // every operand fragment is read once (the products only start after all
    // reads, so no LDS store in between forces a re-read), then the operand
    // copy for the next step is written.
    load_tf(nx, cn);
    const float gn = *reinterpret_cast<const float*>(sg + SM::ST_GN);
    {
      constexpr int JS = SRT >= NWC ? SRT / NWC : 1;  // dk tiles per wave
      constexpr int JT = SUPW / JS;                   // dv tiles per wave
      auto srt_of = [&](int js) { return (wr % SRT) + NWC * js; };
      auto sct_of = [&](int jt) { return SRT >= NWC ? jt : wr / SRT + (NWC / SRT) * jt; };
      frag ka[JS][KCN], vh[JT][KCN], vl[JT][KCN];
#pragma unroll
      for (int js = 0; js < JS; ++js)
#pragma unroll
        for (int kc = 0; kc < KCN; ++kc) {
          const int srt = srt_of(js);
          if constexpr (KROW) {
            ka[js][kc] = load_kt_frag(KT, KP, 32 * kc, 16 * srt, l16, g4);
          } else {
            ka[js][kc] = M::load(KT + (16 * srt + l16) * TP + 32 * kc + 8 * g4);
          }
        }
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int kc = 0; kc < KCN; ++kc) {
          const int o = (16 * sct_of(jt) + l16) * TP + 32 * kc + 8 * g4;
          vh[jt][kc] = M::load(VsT + o);
          if (SPLIT) vl[jt][kc] = M::load(VsL + o);
        }
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int js = 0; js < JS; ++js) {
          const int j = jt * JS + js;  // tile u = wr + NWC j: srt = u % SRT = srt_of(js), sct = u / SRT = sct_of(jt)
          f32x4 acc = Sacc[j] * gn;
#pragma unroll
          for (int kc = 0; kc < KCN; ++kc) {
            acc = M::mma(ka[js][kc], vh[jt][kc], acc);
            if (SPLIT) acc = M::mma(ka[js][kc], vl[jt][kc], acc);
          }
          Sacc[j] = acc;
        }
#pragma unroll
      for (int j = 0; j < SUPW; ++j) {
        const int srt = srt_of(j % JS), sct = sct_of(j / JS);
        M::store4(Sb + (16 * sct + l16) * SP + 16 * srt + 4 * g4, Sacc[j][0], Sacc[j][1], Sacc[j][2], Sacc[j][3]);
      }
    }
    stash(nx, buf ^ 1);  // next step's group-shared operands (its slot was last read one step ago)
    __syncthreads();
  };

  bool pq_gave_up = false;  // see kPollLimit
  auto step_read = [&](FR& st, FR& nx, const int s, const int cn) {
    const int c = chunk_at(s);

    // [A] Z^T = S Q^T for this step's outputs (lane (l16, g4) holds
    // Z[token 16 rt + l16][16 ct + 4 g4 + i]); the state copy is stable
    // until the chain waves' phase C
    load_rows(nx.qf, rq, cn);  // raw q of the next chunk
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = wr + NWC * j;
      if (ALL_UNITS || u < RT * NT) {
        const int ct = u / RT, r = rj(j);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
          z = M::mma(M::load(Sb + (16 * ct + l16) * SP + 32 * ks + 8 * g4), st.qf[r][ks], z);
        Zp[j] = z;
      }
    }
    __syncthreads();

    // [B] the next chunk's P fragments (prepared: the chain waves waited for
    // its ready flag in phase A) and, for a bidirectional second visit, the
    // other direction's partial, loaded a step ahead
    load_pf(nx, cn);
    if constexpr (BI) {
      const bool want = s + 1 < NC && !first_visit(s + 1);
      const rsrc_t rp = want ? ro : rnone;
#pragma unroll
      for (int j = 0; j < UPW; ++j) nx.pq[j] = bload16(rp, out_off[rj(j)] + out_at(cn) + ((wr + NWC * j) / RT) * 64);
    }
    __syncthreads();

    // [C] bidirectional second visit: while any of the partial still holds
    // the fill pattern, the other direction has not stored it yet -- re-read
    // it past the L1 cache; then this chunk's outputs
    if constexpr (BI) {
      if (!first_visit(s)) {
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
          // first test outside any loop: a loop that reloads the tested value
          // makes the compiler wait for every load in flight at its head
          if (__any(any_unwritten(st.pq[j])) && !pq_gave_up) {
            const uint32_t off = out_off[rj(j)] + out_at(c) + ((wr + NWC * j) / RT) * 64;
            f32x4 q = st.pq[j];
            int n = 0;
            for (; n < kPollLimit; ++n) {
              __builtin_amdgcn_s_sleep(2);
              q = bload16_fresh(ro, off);
              if (!__any(any_unwritten(q))) break;
            }
            pq_gave_up = n == kPollLimit;
            st.pq[j] = q;
          }
        }
      }
    }
    readout(st, s, true);
    __syncthreads();
  };

  // two operand stages in ping-pong: the loads for step s+1 are in flight
  // while step s computes (past the last step a valid chunk is reloaded)
  if (NC > 0) {
    const int c0 = chunk_at(0);
    if (!reader) {
      FC sA, sB;
      ensure_ready(ready_flag(c0), c0);
      // steps 0 and 1 load chunks 1 and 2 into sB and sA.  These flag loads come
      // first: the loop's first wait for them must find the operand loads below
      // issued after them, as every later iteration does
      sB.rdy = ready_flag(chunk_at(min(1, NC - 1)));
      sA.rdy = ready_flag(chunk_at(min(2, NC - 1)));
      load_coop(sA, c0);
      load_rows(sA.kf, rk, c0);
      load_tf(sA, c0);
      stash(sA, 0);
      __syncthreads();
      int s = 0;
      for (; s + 1 < NC; s += 2) {
        step_chain(sA, sB, s, chunk_at(s + 1));
        step_chain(sB, sA, s + 1, chunk_at(min(s + 2, NC - 1)));
      }
      if (s < NC) step_chain(sA, sB, s, chunk_at(s));
    } else {
      FR sA, sB;
      load_rows(sA.qf, rq, c0);
      __syncthreads();
      load_pf(sA, c0);  // chunk c0's prepared operands: after the chain waves' wait above
      if constexpr (BI) {  // the partial of step 0 (a single-chunk scan's reverse visit)
        const rsrc_t rp = first_visit(0) ? rnone : ro;
#pragma unroll
        for (int j = 0; j < UPW; ++j) sA.pq[j] = bload16(rp, out_off[rj(j)] + out_at(c0) + ((wr + NWC * j) / RT) * 64);
      }
      int s = 0;
      for (; s + 1 < NC; s += 2) {
        step_read(sA, sB, s, chunk_at(s + 1));
        step_read(sB, sA, s + 1, chunk_at(min(s + 2, NC - 1)));
      }
      if (s < NC) step_read(sA, sB, s, chunk_at(s));
    }
  }

  // ---- final state ----
  if (a.state_out && !reader) {
#pragma unroll
    for (int j = 0; j < SUPW; ++j) {
      const int u = wr + NWC * j;
      const int srt = u % SRT, sct = u / SRT;
      const size_t off = sbase + (size_t)(dv0 + 16 * sct + l16) * DK + 16 * srt + 4 * g4;
      *reinterpret_cast<f32x4*>(a.state_out + off) = Sacc[j];
    }
  }
}

template <typename MT, int DK, int C, int NT, bool BI>
hipError_t launch_chain(const ScanArgs& a, int rev_single, hipStream_t stream, hipFuncAttributes* query) {
  if (query) return hipFuncGetAttributes(query, reinterpret_cast<const void*>(&chain_kernel<MT, DK, C, NT, BI>));
  const int ntiles = a.dv / (16 * NT);
  const int nbh = (int)(a.B * a.H);
  const unsigned nblocks = (unsigned)chain_blocks(nbh, a.dv, NT, BI ? 2 : 1);
  hipLaunchKernelGGL((chain_kernel<MT, DK, C, NT, BI>), dim3(nblocks), dim3(64 * ChainWaves<C, NT>::value), 0, stream,
                     a, rev_single, ntiles, nbh);
  return hipGetLastError();
}

#define GDN_INST_CHAIN(MT, DK, C, NT, BI) \
  template hipError_t launch_chain<MT, DK, C, NT, BI>(const ScanArgs&, int, hipStream_t, hipFuncAttributes*);
#define GDN_INST_CHAIN_D(MT, DK, C, NT) GDN_INST_CHAIN(MT, DK, C, NT, false) GDN_INST_CHAIN(MT, DK, C, NT, true)
#define GDN_INST_CHAIN_N(MT, DK, C) GDN_INST_CHAIN_D(MT, DK, C, 1) GDN_INST_CHAIN_D(MT, DK, C, 2)
GDN_INST_CHAIN_N(float, 64, 32)
GDN_INST_CHAIN_N(float, 64, 64)
GDN_INST_CHAIN_N(float, 128, 32)
GDN_INST_CHAIN_N(float, 128, 64)
GDN_INST_CHAIN_N(bf16, 64, 32)
GDN_INST_CHAIN_N(bf16, 64, 64)
GDN_INST_CHAIN_N(bf16, 128, 32)
GDN_INST_CHAIN_N(bf16, 128, 64)
// 16-token chunks (contractions padded to 32 tokens)
GDN_INST_CHAIN_N(float, 64, 16)
GDN_INST_CHAIN_N(float, 128, 16)
GDN_INST_CHAIN_N(bf16, 64, 16)
GDN_INST_CHAIN_N(bf16, 128, 16)
// 128-token chunks: fp32 operands with d = 128 fit 16-column tiles only
GDN_INST_CHAIN_N(float, 64, 128)
GDN_INST_CHAIN_D(float, 128, 128, 1)
GDN_INST_CHAIN_N(bf16, 64, 128)
GDN_INST_CHAIN_N(bf16, 128, 128)

}  // namespace gdn

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
//   O = (e^g rq) * Z + (q^.k^) Vnew + strict(P) Vnew   (self term in fp32)
//   S = e^{g_last} S + (e^{g_last-g} rk * Vnew)^T K    (matrix cores, fp32 accumulate)
//
// which is the chunked form of S_t = a_t S_{t-1}(I - b_t k^_t k^_t^T) +
// b_t v_t k^_t^T, o_t = S_t q^_t (derivation in the preparation kernel).
//
// Bidirectional scans ("Video DeltaNet", "Methodology in Plain English": a
// forward and a backward recurrent state whose readouts are added) run as two
// direction groups of four waves in one workgroup.  At step s the forward
// group handles chunk s and the reverse group chunk NC-1-s, so every chunk is
// visited twice; the first visitor stores its readout, the second adds its
// own after a workgroup barrier.  The sum therefore needs no atomics and no
// inter-workgroup synchronisation, and `out` is written by plain stores only.
//
// Workgroups are numbered so that all value tiles of one (batch, head) land
// on the same XCD (consecutive workgroups are dealt round-robin over the
// eight XCDs), so the tiles share the chunk operands through one L2.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

template <typename MT, int DK, int C, int NT>
struct ChainSmem {
  static constexpr int EP = 16 / (int)sizeof(MT);
  static constexpr int TP = C + EP;   // pitch of token-contiguous rows
  static constexpr int SP = DK + EP;  // pitch of the state copy
  static constexpr int DT = 16 * NT;
  // k tile of the chunk.  bf16: row-major [C][DK + 16] (the transposed
  // operand of the state update is read with transposing LDS reads; the
  // pitch puts the four rows of one such read in distinct bank quarters).
  // fp32: token-contiguous [DK][TP].
  static constexpr bool KROW = sizeof(MT) == 2;
  static constexpr int KP = DK + 16;
  static constexpr int k_elems = KROW ? C * KP : DK * TP;
  // bf16 operands: Vnew and the scaled update vectors are carried as hi + lo
  // bf16 pairs (two products each), so their rounding stays at fp32 level.
  static constexpr bool SPLIT = sizeof(MT) == 2;
  static constexpr int NVT = SPLIT ? 5 : 3;  // token-contiguous value arrays
  static constexpr int per_group = k_elems + NVT * DT * TP + DT * SP;  // elements
};

template <typename MT, int DT, int C>
struct VTile {
  static constexpr int LPR = DT * (int)sizeof(MT) / 16;  // lanes per token row (16 bytes each)
  static constexpr int NVI = (C * LPR + 127) / 128;      // loads per wave (two waves share the tile)
};

// Raw operands of one chunk, loaded a step ahead of their use.  Every wave
// loads its own matrix-core fragments (k, q rows of its token tile and the
// matching rows of the two chunk triangles); the per-token scales, self-term
// weights, chunk decay and the value tile are loaded once per direction group
// by one or two waves (16 distinct bytes per lane) and staged through LDS.
// Loads are unconditional: rows past the end of the sequence are clamped to
// the last token (their gate scales are exactly zero, so they contribute
// nothing) and all masking and conversion happens at the point of use, so a
// prefetch never forces a wait on the memory pipeline.
template <typename MT, int DK, int C, int NT>
struct Stage {
  typedef typename Mma<MT>::frag frag;
  frag kf[DK / 32];
  frag qf[DK / 32];
  frag tf[C / 32];
  frag pf[C / 32];
  float4 csc;                            // wave 0: scales of token `lane`
  float cpd, cgn;                        // wave 1: self-term weight of token `lane`, chunk decay
  f32x4 cv[VTile<MT, 16 * NT, C>::NVI];  // waves 2, 3: 16 raw bytes of the value tile
};

__device__ __forceinline__ bool tri_needed(bool rev, int kc, int rt) {
  // k-chunks (32 tokens) of a 16-row tile that hold strictly-lower (forward)
  // or strictly-upper (reverse) entries
  return rev ? (32 * kc + 31 > 16 * rt) : (32 * kc <= 16 * rt + 15);
}

// Bit masks that keep the strictly-lower (forward) or strictly-upper
// (reverse) elements of a triangle fragment; only the k-chunk that contains
// the diagonal needs one, and it is loop-invariant per lane.
template <typename MT>
struct FragMask {
  static constexpr int NW = (int)(sizeof(typename Mma<MT>::frag) / 4);
  uint32_t m[NW];
  __device__ __forceinline__ void make(int row, int col0, bool upper) {
#pragma unroll
    for (int i = 0; i < NW; ++i) m[i] = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = col0 + e;
      const bool keep = upper ? (col > row) : (col < row);
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

// Transposed k fragment for the state update, read from a row-major bf16 k
// tile in LDS.  The A operand (m = dk row dk0 + l16, k = 32 tokens from tok0)
// holds, in lane (l16, g4), k[tok0 + 8 g4 + j][dk0 + l16] for j = 0..7.
// ds_read_b64_tr_b16 transposes within each 16-lane group: lane i receives
// res[i][e] = src[4e + i/4][i % 4], where src[s] is the four consecutive bf16
// at source lane s's address (lane mapping checked on gfx950).  Source lane s
// therefore points at k[tok + s/4][dk0 + 4 (s % 4)]; two reads give j = 0..3
// and j = 4..7.
__device__ __forceinline__ bf16x8 load_kt_frag(const bf16* krow, int kp, int tok0, int dk0, int l16, int g4) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* base = (lds_char*)(const_cast<bf16*>(krow));
  const int off0 = ((tok0 + 8 * g4 + (l16 >> 2)) * kp + dk0 + 4 * (l16 & 3)) * 2;
  const int off1 = off0 + 4 * kp * 2;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off0));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off1));
  bf16x8 r;
  __builtin_memcpy(&r, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi, 8);
  return r;
}

// Barrier for the four waves of one direction group, on an LDS counter, so
// the forward and reverse groups of a workgroup do not wait for each other.
// Every wave finishes its own LDS traffic (lgkmcnt 0), arrives, and polls
// until all four have arrived for this epoch.  All four waves of a group are
// resident in the same workgroup, so the wait always ends.
// Polls are bounded (kSpinLimit sleeps, far beyond any legitimate wait) so a
// wave can never spin forever.
constexpr int kSpinLimit = 1 << 22;

__device__ __forceinline__ void spin_until_at_least(int* ctr, int target, int order) {
  for (int n = 0; n < kSpinLimit; ++n) {
    const int v = order == __ATOMIC_ACQUIRE
                      ? __hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)
                      : __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (v >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ void group_barrier(int* ctr, int target, int lane) {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  spin_until_at_least(ctr, target, __ATOMIC_RELAXED);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename MT, int DK, int C, int NT, int DIRS>
__global__ __launch_bounds__(256 * DIRS) void chain_kernel(ScanArgs a, int rev_single, int ntiles, int nbh) {
  using M = Mma<MT>;
  using frag = typename M::frag;
  using SM = ChainSmem<MT, DK, C, NT>;
  using F = Stage<MT, DK, C, NT>;
  constexpr int TP = SM::TP, SP = SM::SP, DT = SM::DT;
  using VT = VTile<MT, DT, C>;
  constexpr int RT = C / 16;              // token row tiles per chunk
  constexpr int UPW = (RT * NT + 3) / 4;  // chunk-output tiles per wave
  constexpr int SRT = DK / 16;            // state row tiles (dk)
  constexpr int SUPW = SRT * NT / 4;      // state tiles per wave
  constexpr bool SPLIT = SM::SPLIT;
  constexpr bool ALL_UNITS = (RT * NT) % 4 == 0;
  constexpr int EPV = 16 / (int)sizeof(MT);  // elements per 16 bytes

  __shared__ __align__(16) MT smem[DIRS * SM::per_group];
  // group-shared per-chunk operands, double buffered by step parity
  __shared__ float4 g_sc[DIRS][2][C];
  __shared__ float g_pd[DIRS][2][C];
  __shared__ float g_gn[DIRS][2];
  __shared__ __align__(16) MT g_v[DIRS][2][C * DT];
  // per-group barrier counters and crossing progress: s_prog[g] counts the
  // waves of group g that have completed (and made visible) the readout
  // stores of their first-visitor steps
  __shared__ int s_gbar[2], s_prog[2];

  // XCD-aware numbering: workgroup id -> (chain, value tile)
  const int id = blockIdx.x;
  const int xcd = id & 7, kk = id >> 3;
  const int chain = (kk / ntiles) * 8 + xcd;
  const int tile = kk % ntiles;
  if (chain >= nbh) return;
  const int64_t NC = a.NC, T = a.T, H = a.H;
  const int64_t b = chain / H, h = chain % H;
  const int dv = a.dv;
  const int dv0 = tile * DT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l16 = lane & 15, g4 = lane >> 4;
  const int dg = wave >> 2, w = wave & 3;
  const bool rev = DIRS == 2 ? (dg == 1) : (rev_single != 0);
  const int slot = DIRS == 2 ? dg : 0;
  const int rt = w % RT;

  constexpr bool KROW = SM::KROW;
  constexpr int KP = SM::KP;
  MT* KT = smem + dg * SM::per_group;        // k tile (layout: see ChainSmem)
  MT* XT = KT + SM::k_elems;                 // [DT][TP]  pseudo-values X^T
  MT* VnT = XT + DT * TP;                    // [DT][TP]  Vnew^T (hi part)
  MT* VsT = VnT + DT * TP;                   // [DT][TP]  (scaled Vnew)^T (hi part)
  MT* VnL = VsT + DT * TP;                   // [DT][TP]  lo parts (bf16 operands only)
  MT* VsL = SPLIT ? VnL + DT * TP : VnL;
  MT* Sb = VsT + (SM::NVT - 2) * DT * TP;    // [DT][SP]  state copy (operand type)

  // ---- loop-invariant addressing: per-lane offsets relative to a chunk's
  // first token, scalar per-chunk bases.  The last chunk may be partial; its
  // offsets clamp rows to the last token. ----
  const int n_last = NC > 0 ? (int)(T - (NC - 1) * C) : C;
  const int HD = (int)(H * DK), HV = (int)(H * dv);
  const int64_t CHD = (int64_t)C * HD, CHV = (int64_t)C * HV;
  const MT* kbase = static_cast<const MT*>(a.k) + (b * T * H + h) * DK;
  const MT* qbase = static_cast<const MT*>(a.q) + (b * T * H + h) * DK;
  const MT* vbase = static_cast<const MT*>(a.v) + (b * T * H + h) * dv + dv0;
  float* obase = a.out + (b * T * H + h) * dv + dv0;
  const int kq_row = 16 * rt + l16;
  const int kq_off = kq_row * HD + 8 * g4;
  const int kq_off_last = min(kq_row, n_last - 1) * HD + 8 * g4;
  int v_off[VT::NVI], v_off_last[VT::NVI];
#pragma unroll
  for (int n = 0; n < VT::NVI; ++n) {
    const int idx = min(max(w - 2, 0) * 64 + n * 128 + lane, C * VT::LPR - 1);
    const int row = idx / VT::LPR, part = idx % VT::LPR;
    v_off[n] = row * HV + part * EPV;
    v_off_last[n] = min(row, n_last - 1) * HV + part * EPV;
  }
  const int o_row0 = 16 * rt + 4 * g4;
  int o_off[4], o_off_last[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o_off[i] = (o_row0 + i) * HV + l16;
    o_off_last[i] = min(o_row0 + i, n_last - 1) * HV + l16;
  }
  const int tri_off = kq_row * C + 8 * g4;
  const int kcd = rt / 2;  // k-chunk holding this row tile's diagonal
  FragMask<MT> dmask;
  dmask.make(kq_row, 32 * kcd + 8 * g4, rev);
  const size_t nch = (size_t)a.B * a.H * a.NC;
  const float4* scb = a.sc + (size_t)slot * nch * C + (size_t)chain * NC * C;
  const float* pdb = a.pd + (size_t)chain * NC * C;
  const float* gnb = a.gn + (size_t)slot * nch + (size_t)chain * NC;
  const MT* trib = static_cast<const MT*>(a.tri) + (size_t)chain * NC * C * C + tri_off;
  const MT* pqkb = static_cast<const MT*>(a.pqk) + (size_t)chain * NC * C * C + tri_off;
  float* const trash = a.trash + lane;

  // ---- loaders (issued a step ahead, spread over the phases) ----
  auto load_coop = [&](F& f, int64_t c) {
    const bool last = c == NC - 1;
    if (w == 0) {
      f.csc = scb[c * C + (lane % C)];
    } else if (w == 1) {
      f.cpd = pdb[c * C + (lane % C)];
      f.cgn = gnb[c];
    } else {
      const MT* p = vbase + c * CHV;
#pragma unroll
      for (int n = 0; n < VT::NVI; ++n) f.cv[n] = *reinterpret_cast<const f32x4*>(p + (last ? v_off_last[n] : v_off[n]));
    }
  };
  auto load_rows = [&](frag* dst, const MT* base, int64_t c) {
    const MT* p = base + c * CHD + (c == NC - 1 ? kq_off_last : kq_off);
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) dst[ks] = M::load(p + 32 * ks);
  };
  auto load_tri = [&](F& f, int64_t c) {
    const MT* tp = trib + c * C * C;
    const MT* pp = pqkb + c * C * C;
#pragma unroll
    for (int kc = 0; kc < C / 32; ++kc) {
      if (tri_needed(rev, kc, rt)) {  // wave-uniform
        f.tf[kc] = M::load(tp + 32 * kc);
        f.pf[kc] = M::load(pp + 32 * kc);
      }
    }
  };
  auto stash = [&](const F& f, int buf) {  // group-shared registers of a loaded stage -> LDS slot
    if (w == 0) {
      if (lane < C) g_sc[dg][buf][lane] = f.csc;
    } else if (w == 1) {
      if (lane < C) g_pd[dg][buf][lane] = f.cpd;
      if (lane == 0) g_gn[dg][buf] = f.cgn;
    } else {
#pragma unroll
      for (int n = 0; n < VT::NVI; ++n) {
        const int idx = (w - 2) * 64 + n * 128 + lane;
        if (idx < C * VT::LPR) *reinterpret_cast<f32x4*>(&g_v[dg][buf][idx * EPV]) = f.cv[n];
      }
    }
  };
  // output element (row o_row0+i, column tile of unit j) of chunk c
  auto out_at = [&](int64_t c, int j, int i) -> float* {
    const int ct = (w + 4 * j) / RT;
    return obase + c * CHV + (c == NC - 1 ? o_off_last[i] : o_off[i]) + 16 * ct;
  };
  auto row_valid = [&](int64_t c, int i) { return o_row0 + i < (c == NC - 1 ? n_last : C); };

  if (threadIdx.x == 0) {
    s_gbar[0] = s_gbar[1] = 0;
    s_prog[0] = s_prog[1] = 0;
  }
  int epoch = 0;  // group barriers passed (wave-uniform)
  auto gsync = [&]() {
    if (DIRS == 1) {
      __syncthreads();
    } else {
      ++epoch;
      group_barrier(&s_gbar[dg], 4 * epoch, lane);
    }
  };

  // ---- initial state into accumulators (S^T tiles) and the operand copy ----
  f32x4 Sacc[SUPW];
  const size_t sbase = (((size_t)slot * a.B + b) * a.H + h) * (size_t)dv * DK;
#pragma unroll
  for (int j = 0; j < SUPW; ++j) {
    const int u = w + 4 * j;
    const int srt = u % SRT, sct = u / SRT;
    const size_t off = sbase + (size_t)(dv0 + 16 * sct + l16) * DK + 16 * srt + 4 * g4;
    Sacc[j] = a.state_in ? *reinterpret_cast<const f32x4*>(a.state_in + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    M::store4(Sb + (16 * sct + l16) * SP + 16 * srt + 4 * g4, Sacc[j][0], Sacc[j][1], Sacc[j][2], Sacc[j][3]);
  }

  // The other direction's readout of the chunk of step s, if it was stored
  // in an earlier step.  A first visitor stores in the last phase of its
  // step, so these loads are issued after the first barrier of step s (which
  // orders them after every store of step s-1 and earlier), and before the
  // next stage's remaining loads: the memory counter retires in order.
  float part[UPW][4];
  auto chunk_at = [&](int64_t s) { return rev ? NC - 1 - s : s; };
  auto load_part = [&](int64_t s) {
    if (DIRS == 2) {
      const int64_t so = NC - 1 - s;
      const bool second = s > so || (s == so && rev);
      if (second) {  // the other group stored this chunk in its step so: wait for it
        spin_until_at_least(&s_prog[1 - dg], 4 * (int)(so + 1), __ATOMIC_ACQUIRE);
      }
      const int64_t c = chunk_at(s);
#pragma unroll
      for (int j = 0; j < UPW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[j][i] = *out_at(c, j, i);
    }
  };

  auto step = [&](F& st, F& nx, int64_t s, int64_t cn) {
    const int64_t c = chunk_at(s);
    const int64_t so = NC - 1 - s;  // step at which the other direction visits chunk c
    const bool first = DIRS == 1 || s < so || (s == so && !rev);
    const int buf = (int)(s & 1);
    float4 sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = g_sc[dg][buf][o_row0 + i];

    // [A] k tile into LDS; Y = K S^T, Z = Q S^T; X
    if (w < RT) {
      if constexpr (KROW) {
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
          *reinterpret_cast<frag*>(KT + kq_row * KP + 32 * ks + 8 * g4) = st.kf[ks];
      } else {
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            KT[(32 * ks + 8 * g4 + e) * TP + kq_row] = (MT)M::get(st.kf[ks], e);
      }
    }
    load_rows(nx.kf, kbase, cn);
    f32x4 X[UPW], Z[UPW], Vn[UPW];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = w + 4 * j;
      if (ALL_UNITS || u < RT * NT) {
        const int ct = u / RT;
        f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const frag sb = M::load(Sb + (16 * ct + l16) * SP + 32 * ks + 8 * g4);
          y = M::mma(st.kf[ks], sb, y);
          z = M::mma(st.qf[ks], sb, z);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          X[j][i] = sc[i].x * (to_f32(g_v[dg][buf][(o_row0 + i) * DT + 16 * ct + l16]) - sc[i].y * y[i]);
        Z[j] = z;
        M::store4(XT + (16 * ct + l16) * TP + o_row0, X[j][0], X[j][1], X[j][2], X[j][3]);
      }
    }
    gsync();

    // [B] Vnew = X + strict(Tinv) X
    load_part(s);
    load_rows(nx.qf, qbase, cn);
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = w + 4 * j;
      if (ALL_UNITS || u < RT * NT) {
        const int ct = u / RT;
        f32x4 acc = X[j];
#pragma unroll
        for (int kc = 0; kc < C / 32; ++kc) {
          if (tri_needed(rev, kc, rt)) {
            const frag tf = kc == kcd ? dmask.apply(st.tf[kc]) : st.tf[kc];
            acc = M::mma(tf, M::load(XT + (16 * ct + l16) * TP + 32 * kc + 8 * g4), acc);
          }
        }
        Vn[j] = acc;
        const int o = (16 * ct + l16) * TP + o_row0;
        f32x4 vs;
#pragma unroll
        for (int i = 0; i < 4; ++i) vs[i] = sc[i].w * acc[i];
        M::store4(VnT + o, acc[0], acc[1], acc[2], acc[3]);
        M::store4(VsT + o, vs[0], vs[1], vs[2], vs[3]);
        if (SPLIT) {
          f32x4 rn, rs;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            rn[i] = acc[i] - (float)(MT)acc[i];
            rs[i] = vs[i] - (float)(MT)vs[i];
          }
          M::store4(VnL + o, rn[0], rn[1], rn[2], rn[3]);
          M::store4(VsL + o, rs[0], rs[1], rs[2], rs[3]);
        }
      }
    }
    gsync();

    // [C] chunk readout (a causal scan stores it right away)
    load_tri(nx, cn);
    f32x4 O[UPW];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = w + 4 * j;
      if (ALL_UNITS || u < RT * NT) {
        const int ct = u / RT;
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = sc[i].z * Z[j][i] + g_pd[dg][buf][o_row0 + i] * Vn[j][i];
#pragma unroll
        for (int kc = 0; kc < C / 32; ++kc) {
          if (tri_needed(rev, kc, rt)) {
            const frag pf = kc == kcd ? dmask.apply(st.pf[kc]) : st.pf[kc];
            const int o = (16 * ct + l16) * TP + 32 * kc + 8 * g4;
            acc = M::mma(pf, M::load(VnT + o), acc);
            if (SPLIT) acc = M::mma(pf, M::load(VnL + o), acc);
          }
        }
        O[j] = acc;
        if (DIRS == 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) *(row_valid(c, i) ? out_at(c, j, i) : trash) = acc[i];
        }
      }
    }
    // state update S^T = gn S^T + K^T Vs
    const float gn = g_gn[dg][buf];
#pragma unroll
    for (int j = 0; j < SUPW; ++j) {
      const int u = w + 4 * j;
      const int srt = u % SRT, sct = u / SRT;
      f32x4 acc = Sacc[j] * gn;
#pragma unroll
      for (int kc = 0; kc < C / 32; ++kc) {
        frag ka;
        if constexpr (KROW) {
          ka = load_kt_frag(KT, KP, 32 * kc, 16 * srt, l16, g4);
        } else {
          ka = M::load(KT + (16 * srt + l16) * TP + 32 * kc + 8 * g4);
        }
        const int o = (16 * sct + l16) * TP + 32 * kc + 8 * g4;
        acc = M::mma(ka, M::load(VsT + o), acc);
        if (SPLIT) acc = M::mma(ka, M::load(VsL + o), acc);
      }
      Sacc[j] = acc;
      M::store4(Sb + (16 * sct + l16) * SP + 16 * srt + 4 * g4, acc[0], acc[1], acc[2], acc[3]);
    }
    stash(nx, buf ^ 1);  // next step's group-shared operands (its slot was last read one step ago)
    gsync();

    // [D] bidirectional: the first visitor stores its readout, the second
    // adds its own to the one stored by the other group (loaded in [B]).  A
    // first visitor then makes its stores visible and counts its progress.
    if (DIRS == 2) {
#pragma unroll
      for (int j = 0; j < UPW; ++j) {
        if (ALL_UNITS || w + 4 * j < RT * NT) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *(row_valid(c, i) ? out_at(c, j, i) : trash) = O[j][i] + (first ? 0.f : part[j][i]);
        }
      }
      if (first) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_fetch_add(&s_prog[dg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  };

  // two operand stages in ping-pong: the loads for step s+1 are in flight
  // while step s computes (past the last step a valid chunk is reloaded)
  F sA, sB;
  if (NC > 0) {
    const int64_t c0 = chunk_at(0);
    load_coop(sA, c0);
    load_rows(sA.kf, kbase, c0);
    load_rows(sA.qf, qbase, c0);
    load_tri(sA, c0);
    stash(sA, 0);
    __syncthreads();
    for (int64_t s = 0; s < NC; s += 2) {
      const int64_t c1 = chunk_at(min(s + 1, NC - 1));
      load_coop(sB, c1);
      step(sA, sB, s, c1);
      if (s + 1 < NC) {
        const int64_t c2 = chunk_at(min(s + 2, NC - 1));
        load_coop(sA, c2);
        step(sB, sA, s + 1, c2);
      }
    }
  } else {
    __syncthreads();
  }

  // ---- final state ----
  if (a.state_out) {
#pragma unroll
    for (int j = 0; j < SUPW; ++j) {
      const int u = w + 4 * j;
      const int srt = u % SRT, sct = u / SRT;
      const size_t off = sbase + (size_t)(dv0 + 16 * sct + l16) * DK + 16 * srt + 4 * g4;
      *reinterpret_cast<f32x4*>(a.state_out + off) = Sacc[j];
    }
  }
}

template <typename MT, int DK, int C, int NT, int DIRS>
hipError_t launch_chain(const ScanArgs& a, int rev_single, hipStream_t stream) {
  const int ntiles = a.dv / (16 * NT);
  const int nbh = (int)(a.B * a.H);
  const int groups = (nbh + 7) / 8;
  const unsigned nblocks = (unsigned)(groups * 8 * ntiles);
  hipLaunchKernelGGL((chain_kernel<MT, DK, C, NT, DIRS>), dim3(nblocks), dim3(256 * DIRS), 0, stream, a,
                     rev_single, ntiles, nbh);
  return hipGetLastError();
}

#define GDN_INST_CHAIN(MT, DK, C, NT, DIRS) \
  template hipError_t launch_chain<MT, DK, C, NT, DIRS>(const ScanArgs&, int, hipStream_t);
#define GDN_INST_CHAIN_D(MT, DK, C, NT) GDN_INST_CHAIN(MT, DK, C, NT, 1) GDN_INST_CHAIN(MT, DK, C, NT, 2)
#define GDN_INST_CHAIN_N(MT, DK, C) GDN_INST_CHAIN_D(MT, DK, C, 1) GDN_INST_CHAIN_D(MT, DK, C, 2)
GDN_INST_CHAIN_N(float, 64, 32)
GDN_INST_CHAIN_N(float, 64, 64)
GDN_INST_CHAIN_N(float, 128, 32)
GDN_INST_CHAIN_D(float, 128, 64, 1)  // fp32, dk 128, 32-wide tiles: exceeds LDS
GDN_INST_CHAIN_N(bf16, 64, 32)
GDN_INST_CHAIN_N(bf16, 64, 64)
GDN_INST_CHAIN_N(bf16, 128, 32)
GDN_INST_CHAIN_N(bf16, 128, 64)

}  // namespace gdn

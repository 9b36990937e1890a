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
  // bf16 operands: Vnew and the scaled update vectors are carried as hi + lo
  // bf16 pairs (two products each), so their rounding stays at fp32 level.
  static constexpr bool SPLIT = sizeof(MT) == 2;
  static constexpr int NVT = SPLIT ? 5 : 3;  // token-contiguous value arrays
  static constexpr int per_group = DK * TP + NVT * DT * TP + DT * SP;  // elements
};

template <typename MT, int DK, int C, int NT>
struct ChunkFrags {
  typedef typename Mma<MT>::frag frag;
  frag kf[DK / 32];
  frag qf[DK / 32];
  frag tf[C / 32];
  frag pf[C / 32];
  float4 sc[4];
  float pd[4];
  float v[NT][4];
  float gn;
};

template <typename MT, int DK, int C, int NT>
__device__ __forceinline__ void load_chunk(ChunkFrags<MT, DK, C, NT>& f, const ScanArgs& a, int64_t b, int64_t h,
                                           int64_t chain, int64_t c, int slot, bool rev, int rt, int w, int dv0,
                                           int l16, int g4) {
  using M = Mma<MT>;
  constexpr int RT = C / 16;
  const int64_t T = a.T, H = a.H;
  const int64_t t0 = c * C;
  const int64_t cid = chain * a.NC + c;
  const MT* k = static_cast<const MT*>(a.k);
  const MT* q = static_cast<const MT*>(a.q);
  const MT* v = static_cast<const MT*>(a.v);
  {
    const int64_t t = t0 + 16 * rt + l16;
    const bool valid = t < T;
    const int64_t off = ((b * T + (valid ? t : 0)) * H + h) * DK + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      f.kf[ks] = load_frag_global<MT>(k + off + 32 * ks, valid);
      f.qf[ks] = load_frag_global<MT>(q + off + 32 * ks, valid);
    }
  }
  {
    const MT* tri = static_cast<const MT*>(a.tri) + cid * C * C;
    const MT* pqk = static_cast<const MT*>(a.pqk) + cid * C * C;
    const int row = 16 * rt + l16;
#pragma unroll
    for (int kc = 0; kc < C / 32; ++kc) {
      const bool need = rev ? (32 * kc + 31 > 16 * rt) : (32 * kc <= 16 * rt + 15);
      if (need) {
        const int col0 = 32 * kc + 8 * g4;
        f.tf[kc] = mask_tri<MT>(M::load(tri + row * C + col0), row, col0, rev);
        f.pf[kc] = mask_tri<MT>(M::load(pqk + row * C + col0), row, col0, rev);
      } else {
        f.tf[kc] = M::zero();
        f.pf[kc] = M::zero();
      }
    }
  }
  const size_t nch = (size_t)a.B * a.H * a.NC;
  const float4* sc = a.sc + (size_t)slot * nch * C + cid * C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * rt + 4 * g4 + i;
    f.sc[i] = sc[r];
    f.pd[i] = a.pd[cid * C + r];
    const int64_t t = t0 + r;
    const bool valid = t < T;
    const int64_t voff = ((b * T + (valid ? t : 0)) * H + h) * a.dv + dv0 + l16;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int u = w + 4 * j;
      const int ct = u / RT;
      f.v[j][i] = (valid && u < RT * NT) ? to_f32(v[voff + 16 * ct]) : 0.f;
    }
  }
  f.gn = a.gn[(size_t)slot * nch + cid];
}

template <typename MT, int DK, int C, int NT, int DIRS>
__global__ __launch_bounds__(256 * DIRS) void chain_kernel(ScanArgs a, int rev_single, int ntiles, int nbh) {
  using M = Mma<MT>;
  using SM = ChainSmem<MT, DK, C, NT>;
  using F = ChunkFrags<MT, DK, C, NT>;
  constexpr int TP = SM::TP, SP = SM::SP, DT = SM::DT;
  constexpr int RT = C / 16;            // token row tiles per chunk
  constexpr int UPW = (RT * NT + 3) / 4;  // chunk-output tiles per wave
  constexpr int SRT = DK / 16;          // state row tiles (dk)
  constexpr int SUPW = SRT * NT / 4;    // state tiles per wave

  __shared__ __align__(16) MT smem[DIRS * SM::per_group];

  // XCD-aware numbering: workgroup id -> (chain, value tile)
  const int id = blockIdx.x;
  const int xcd = id & 7, kk = id >> 3;
  const int chain = (kk / ntiles) * 8 + xcd;
  const int tile = kk % ntiles;
  if (chain >= nbh) return;
  const int64_t b = chain / a.H, h = chain % a.H;
  const int dv0 = tile * DT;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int dg = wave / 4, w = wave % 4;
  const bool rev = DIRS == 2 ? (dg == 1) : (rev_single != 0);
  const int slot = DIRS == 2 ? dg : 0;
  const int rt = w % RT;
  const int64_t NC = a.NC, T = a.T;
  const int dv = a.dv;

  constexpr bool SPLIT = SM::SPLIT;
  MT* KT = smem + dg * SM::per_group;        // [DK][TP]  k, token-contiguous
  MT* XT = KT + DK * TP;                     // [DT][TP]  pseudo-values X^T
  MT* VnT = XT + DT * TP;                    // [DT][TP]  Vnew^T (hi part)
  MT* VsT = VnT + DT * TP;                   // [DT][TP]  (scaled Vnew)^T (hi part)
  MT* VnL = VsT + DT * TP;                   // [DT][TP]  lo parts (bf16 operands only)
  MT* VsL = SPLIT ? VnL + DT * TP : VnL;
  MT* Sb = VsT + (SM::NVT - 2) * DT * TP;    // [DT][SP]  state copy (operand type)

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
  __syncthreads();

  F cur, nxt;
  if (NC > 0) load_chunk<MT, DK, C, NT>(cur, a, b, h, chain, rev ? NC - 1 : 0, slot, rev, rt, w, dv0, l16, g4);

  for (int64_t s = 0; s < NC; ++s) {
    const int64_t c = rev ? NC - 1 - s : s;
    const int64_t t0 = c * C;
    if (s + 1 < NC) load_chunk<MT, DK, C, NT>(nxt, a, b, h, chain, rev ? c - 1 : c + 1, slot, rev, rt, w, dv0, l16, g4);

    // [A] k into the token-contiguous layout; Y, Z; pseudo-values X
    if (w < RT) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          KT[(32 * ks + 8 * g4 + e) * TP + 16 * rt + l16] = (MT)M::get(cur.kf[ks], e);
    }
    f32x4 X[UPW], Z[UPW], Vn[UPW];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = w + 4 * j;
      if (u < RT * NT) {
        const int ct = u / RT;
        f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const typename M::frag sb = M::load(Sb + (16 * ct + l16) * SP + 32 * ks + 8 * g4);
          y = M::mma(cur.kf[ks], sb, y);
          z = M::mma(cur.qf[ks], sb, z);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) X[j][i] = cur.sc[i].x * (cur.v[j][i] - cur.sc[i].y * y[i]);
        Z[j] = z;
        M::store4(XT + (16 * ct + l16) * TP + 16 * rt + 4 * g4, X[j][0], X[j][1], X[j][2], X[j][3]);
      }
    }
    __syncthreads();

    // [B] Vnew = X + strict(Tinv) X
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = w + 4 * j;
      if (u < RT * NT) {
        const int ct = u / RT;
        f32x4 acc = X[j];
#pragma unroll
        for (int kc = 0; kc < C / 32; ++kc) {
          const bool need = rev ? (32 * kc + 31 > 16 * rt) : (32 * kc <= 16 * rt + 15);
          if (need) acc = M::mma(cur.tf[kc], M::load(XT + (16 * ct + l16) * TP + 32 * kc + 8 * g4), acc);
        }
        Vn[j] = acc;
        const int o = (16 * ct + l16) * TP + 16 * rt + 4 * g4;
        f32x4 vs;
#pragma unroll
        for (int i = 0; i < 4; ++i) vs[i] = cur.sc[i].w * acc[i];
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
    __syncthreads();

    // [C] chunk readout; first visitor (or causal) stores it
    const bool first = DIRS == 1 ? true : (rev ? (2 * c > NC - 1) : (2 * c <= NC - 1));
    f32x4 O[UPW];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = w + 4 * j;
      if (u < RT * NT) {
        const int ct = u / RT;
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = cur.sc[i].z * Z[j][i] + cur.pd[i] * Vn[j][i];
#pragma unroll
        for (int kc = 0; kc < C / 32; ++kc) {
          const bool need = rev ? (32 * kc + 31 > 16 * rt) : (32 * kc <= 16 * rt + 15);
          if (need) {
            const int o = (16 * ct + l16) * TP + 32 * kc + 8 * g4;
            acc = M::mma(cur.pf[kc], M::load(VnT + o), acc);
            if (SPLIT) acc = M::mma(cur.pf[kc], M::load(VnL + o), acc);
          }
        }
        O[j] = acc;
        if (first) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + 16 * rt + 4 * g4 + i;
            if (t < T) a.out[((b * T + t) * a.H + h) * dv + dv0 + 16 * ct + l16] = acc[i];
          }
        }
      }
    }
    // state update S^T = gn S^T + K^T Vs
#pragma unroll
    for (int j = 0; j < SUPW; ++j) {
      const int u = w + 4 * j;
      const int srt = u % SRT, sct = u / SRT;
      f32x4 acc = Sacc[j] * cur.gn;
#pragma unroll
      for (int kc = 0; kc < C / 32; ++kc) {
        const typename M::frag ka = M::load(KT + (16 * srt + l16) * TP + 32 * kc + 8 * g4);
        const int o = (16 * sct + l16) * TP + 32 * kc + 8 * g4;
        acc = M::mma(ka, M::load(VsT + o), acc);
        if (SPLIT) acc = M::mma(ka, M::load(VsL + o), acc);
      }
      Sacc[j] = acc;
      M::store4(Sb + (16 * sct + l16) * SP + 16 * srt + 4 * g4, acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();

    // [D] second visitor adds its readout to the stored one
    if (!first) {
#pragma unroll
      for (int j = 0; j < UPW; ++j) {
        const int u = w + 4 * j;
        if (u < RT * NT) {
          const int ct = u / RT;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + 16 * rt + 4 * g4 + i;
            if (t < T) {
              float* p = a.out + ((b * T + t) * a.H + h) * dv + dv0 + 16 * ct + l16;
              *p = *p + O[j][i];
            }
          }
        }
      }
    }
    if (s + 1 < NC) cur = nxt;
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
GDN_INST_CHAIN_N(float, 128, 64)
GDN_INST_CHAIN_N(bf16, 64, 32)
GDN_INST_CHAIN_N(bf16, 64, 64)
GDN_INST_CHAIN_N(bf16, 128, 32)
GDN_INST_CHAIN_N(bf16, 128, 64)

}  // namespace gdn

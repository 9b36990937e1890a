// Chunk preparation kernel: everything of the chunked scan that does not
// depend on the recurrent state.
//
// The recurrence S_t = a_t S_{t-1}(I - b_t k^_t k^_t^T) + b_t v_t k^_t^T can be
// evaluated C tokens at a time.  The pages name the ingredients -- chunk-wise
// scans and a fused blocked small-matrix inverse that stays on chip ("Video
// DeltaNet", "Key Contributions" item 4 and "Main Findings", kernel
// optimisations) -- and the chunk equations follow from the recurrence.  For
// a chunk entered with state S (processing order r = 0..n-1):
//
//   g_r = sum_{j<=r} log_alpha_j,   Gam_ri = exp(g_r - g_i) (i <= r)
//   L   = strictly_lower(diag(beta) (K^ K^^T) * Gam),   Tinv = (I + L)^{-1}
//   X   = diag(beta)(V - diag(e^g) K^ S^T),   Vnew = Tinv X
//   O   = diag(e^g) Q^ S^T + ((Q^ K^^T) * Gam) Vnew
//   S'  = e^{g_last} S + Vnew^T diag(e^{g_last - g}) K^
//
// This kernel produces, per (batch, head, chunk), the state-independent
// pieces: Tinv and the decayed Q^K^^T for both directions (the forward one
// in the strictly-lower triangle, the reverse one -- the same recurrence with
// tokens visited last-to-first -- in the strictly-upper triangle, both in
// natural token order, with the self terms q^_t.k^_t on the shared diagonal
// of Q^K^^T), the per-token gate scales and the chunk decays.  One Gram matrix
// K K^T serves both directions.
//
// Normalisation is never applied to the operands: K K^T and Q K^T are taken
// on the raw inputs on the matrix cores (fp32 accumulation) and the fp32 row
// scales rk = 1/max(|k|, eps), rq = 1/max(|q|, eps) are applied afterwards.
//
// The unit-triangular inverse is blocked in 16 x 16 tiles in LDS (fp32): the
// diagonal tiles are inverted by substitution (one column per thread), then
// each column of off-diagonal tiles follows from T_IJ = -T_II sum_K L_IK T_KJ
// on the fp32 matrix cores.  A block column only depends on itself and on
// the diagonal tiles, so each column is one wave's private chain.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

template <typename MT, int DK, int C>
struct PrepSmem {
  static constexpr int EP = 16 / (int)sizeof(MT);       // elements per 16-byte piece
  static constexpr int KP = DK + EP;                    // padded row pitch of staged q/k
  static constexpr int NB = C / 16;                     // 16 x 16 blocks per side
  static constexpr int LP = C + 1;                      // pitch of fp32 C x C tiles
  static constexpr int PP = C + EP;                     // pitch of the staged decayed q.k tile
  static constexpr size_t kq_bytes = (size_t)2 * C * KP * sizeof(MT);
  static constexpr size_t inv_bytes = (size_t)2 * C * LP * 4 + (size_t)C * PP * sizeof(MT) + (size_t)4 * 16 * 17 * 4;
  static constexpr size_t region = kq_bytes > inv_bytes ? kq_bytes : inv_bytes;
};

template <typename MT, int DK, int C>
__global__ __launch_bounds__(256) void chunk_prep_kernel(ScanArgs a) {
  using SM = PrepSmem<MT, DK, C>;
  using M = Mma<MT>;
  constexpr int EP = SM::EP, KP = SM::KP, NB = SM::NB, LP = SM::LP;

  __shared__ __align__(16) unsigned char smem[SM::region];
  __shared__ float s_rk[C], s_rq[C];
  __shared__ float s_la[2][C], s_bt[2][C], s_g[2][C];

  constexpr int PP = SM::PP;
  MT* Ks = reinterpret_cast<MT*>(smem);
  MT* Qs = Ks + C * KP;
  float* Lm = reinterpret_cast<float*>(smem);  // reused after the Gram products
  float* Ti = Lm + C * LP;
  MT* Pst = reinterpret_cast<MT*>(Ti + C * LP);                          // decayed q.k, staged
  float* Wsc = reinterpret_cast<float*>(Pst + C * PP);                   // [4 waves][16][17]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t T = a.T, H = a.H, B = a.B;
  const int64_t t0 = c * C;
  const int64_t cid = bh * a.NC + c;
  const int fwd_on = a.fwd_on, rev_on = a.rev_on;
  const int fslot = 0, rslot = fwd_on ? 1 : 0;
  const size_t nch = (size_t)a.B * a.H * a.NC;

  // ---- stage raw q and k of this chunk into LDS (padded rows are zero) ----
  {
    const MT* q = static_cast<const MT*>(a.q);
    const MT* k = static_cast<const MT*>(a.k);
    constexpr int PR = DK / EP;  // pieces per row
    constexpr int NP = C * PR;   // pieces per matrix
#pragma unroll
    for (int p = tid; p < NP; p += 256) {
      const int row = p / PR, cp = (p % PR) * EP;
      const int64_t t = t0 + row;
      f32x4 vq = {0.f, 0.f, 0.f, 0.f}, vk = {0.f, 0.f, 0.f, 0.f};
      if (t < T) {
        const int64_t off = ((b * T + t) * H + h) * DK + cp;
        vq = *reinterpret_cast<const f32x4*>(q + off);
        vk = *reinterpret_cast<const f32x4*>(k + off);
      }
      *reinterpret_cast<f32x4*>(Qs + row * KP + cp) = vq;
      *reinterpret_cast<f32x4*>(Ks + row * KP + cp) = vk;
    }
  }
  if (tid < C) {
    const int64_t t = t0 + tid;
    const bool in = t < T;
    if (fwd_on) {
      const int64_t gi = ((fslot * B + b) * T + t) * H + h;
      s_la[0][tid] = in ? a.log_alpha[gi] : 0.f;
      s_bt[0][tid] = in ? a.beta[gi] : 0.f;
    }
    if (rev_on) {
      const int64_t gi = ((rslot * B + b) * T + t) * H + h;
      s_la[1][tid] = in ? a.log_alpha[gi] : 0.f;
      s_bt[1][tid] = in ? a.beta[gi] : 0.f;
    }
  }
  __syncthreads();

  // ---- row scales and chunk-local cumulative log-gates ----
  {
    constexpr int G = 256 / C;        // threads per row
    constexpr int PER = DK / G;       // elements per thread (a multiple of 8)
    const int row = tid / G, part = tid % G;
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e8 = 0; e8 < PER; e8 += 8) {  // 8 elements per fragment-sized read
      const typename M::frag fq = M::load(Qs + row * KP + part * PER + e8);
      const typename M::frag fk = M::load(Ks + row * KP + part * PER + e8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xq = M::get(fq, e), xk = M::get(fk, e);
        sq = fmaf(xq, xq, sq);
        sk = fmaf(xk, xk, sk);
      }
    }
#pragma unroll
    for (int m = 1; m < G; m <<= 1) {
      sq += __shfl_xor(sq, m, 64);
      sk += __shfl_xor(sk, m, 64);
    }
    if (part == 0) {
      s_rq[row] = 1.0f / fmaxf(sqrtf(sq), kNormEps);
      s_rk[row] = 1.0f / fmaxf(sqrtf(sk), kNormEps);
    }
  }
  // chunk-local cumulative log-gates, kept in log2 units so every decay
  // factor below is one exp2 of a difference: wave 0 forms the inclusive
  // prefix sums in token order, wave 1 the inclusive suffix sums (the reverse
  // visiting order), each as a wave-wide scan
  constexpr float kLog2e = 1.4426950408889634f;
  if (wave < 2 && (wave == 0 ? fwd_on : rev_on)) {
    const int dir = wave;
    const int tok = dir == 0 ? lane : C - 1 - lane;  // position in visiting order = lane
    float s = lane < C ? s_la[dir][tok] : 0.f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float o = __shfl_up(s, d, 64);
      if (lane >= d) s += o;
    }
    if (lane < C) s_g[dir][tok] = s * kLog2e;
  }
  __syncthreads();

  // ---- Gram K K^T and Q K^T on the matrix cores (raw operands, fp32 accumulate) ----
  constexpr int NT2 = NB * NB;
  constexpr int UPW = (NT2 + 3) / 4;
  f32x4 accG[UPW], accP[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    accG[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    accP[j] = accG[j];
    const int u = wave + 4 * j;
    if (u < NT2) {
      const int ti = u / NB, tj = u % NB;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const typename M::frag ka = M::load(Ks + (16 * ti + l16) * KP + 32 * ks + 8 * g4);
        const typename M::frag qa = M::load(Qs + (16 * ti + l16) * KP + 32 * ks + 8 * g4);
        const typename M::frag kb = M::load(Ks + (16 * tj + l16) * KP + 32 * ks + 8 * g4);
        accG[j] = M::mma(ka, kb, accG[j]);
        accP[j] = M::mma(qa, kb, accP[j]);
      }
    }
  }
  __syncthreads();  // q/k staging area is reused below

  // ---- gated, scaled triangles: L and the decayed Q^K^^T into LDS ----
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = wave + 4 * j;
    if (u < NT2) {
      const int ti = u / NB, tj = u % NB;
      const int col = 16 * tj + l16;
      const float rkc = s_rk[col];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * ti + 4 * g4 + i;
        float lv = 0.f, pv = 0.f;
        if (col < r) {
          if (fwd_on) {
            const float gam = exp2f(s_g[0][r] - s_g[0][col]);
            lv = s_bt[0][r] * s_rk[r] * rkc * accG[j][i] * gam;
            pv = s_rq[r] * rkc * accP[j][i] * gam;
          }
        } else if (col > r) {
          if (rev_on) {
            const float gam = exp2f(s_g[1][r] - s_g[1][col]);
            lv = s_bt[1][r] * s_rk[r] * rkc * accG[j][i] * gam;
            pv = s_rq[r] * rkc * accP[j][i] * gam;
          }
        } else {
          // self term q^_r . k^_r: on the diagonal in the operand type, the
          // remainder that type drops into each direction's record
          pv = s_rq[r] * s_rk[r] * accP[j][i];
          const float lo = pv - (float)(MT)pv;
          if (fwd_on) a.pdg[((size_t)fslot * nch + cid) * (C + 4) + r] = lo;
          if (rev_on) a.pdg[((size_t)rslot * nch + cid) * (C + 4) + r] = lo;
        }
        Lm[r * LP + col] = lv;
        Pst[r * PP + col] = (MT)pv;
      }
    }
  }
  __syncthreads();

  // ---- diagonal 16 x 16 blocks: one column of the inverse per thread ----
  if (tid < 2 * NB * 16) {
    const int dir = tid / (NB * 16);
    const int blk = (tid / 16) % NB;
    const int jc = tid % 16;
    const int b0 = 16 * blk;
    // column jc of (I + L_bb)^{-1} by forward substitution in visiting
    // order, column-oriented: once x_i is known it is folded into every
    // later row's running sum, so the dependent chain is 16 steps long.
    // One instance per direction keeps every index a compile-time constant
    // (the running sums stay in registers).
    auto solve = [&](auto rev_tag) {
      constexpr bool R = decltype(rev_tag)::value;
      float acc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int i = R ? 15 - ii : ii;  // visiting order
        const bool after = R ? (i < jc) : (i > jc);
        const float x = i == jc ? 1.f : (after ? -acc[i] : 0.f);
        if (i == jc || after) Ti[(b0 + i) * LP + b0 + jc] = x;
#pragma unroll
        for (int rr = ii + 1; rr < 16; ++rr) {
          const int r = R ? 15 - rr : rr;
          acc[r] = fmaf(Lm[(b0 + r) * LP + b0 + i], x, acc[r]);
        }
      }
    };
    if (dir == 0 && fwd_on) solve(std::false_type{});
    if (dir == 1 && rev_on) solve(std::true_type{});
  }
  __syncthreads();

  // ---- off-diagonal blocks: one block column per wave, on fp32 matrix cores ----
  // v_mfma_f32_16x16x4f32: lane (l16, g4) supplies A[l16][k] and B[k][l16]
  // with k = 4 ks + g4; D lands as D[4 g4 + i][l16].
  {
    float* wsc = Wsc + wave * 16 * 17;
    auto column = [&](int dir, int J) {
      const bool up = dir == 1;
      const int I0 = up ? J - 1 : J + 1;
      const int I1 = up ? -1 : NB;
      const int dI = up ? -1 : 1;
      for (int I = I0; I != I1; I += dI) {
        // W = sum_K L_IK T_KJ over K between J and I (T_JJ triangular)
        f32x4 w = {0.f, 0.f, 0.f, 0.f};
        const int K0 = up ? I + 1 : J, K1 = up ? J : I - 1;
        for (int K = K0; K <= K1; ++K) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int k = 4 * ks + g4;
            const float av = Lm[(16 * I + l16) * LP + 16 * K + k];
            float bv = Ti[(16 * K + k) * LP + 16 * J + l16];
            if (K == J && (up ? k > l16 : k < l16)) bv = 0.f;
            w = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, w, 0, 0, 0);
          }
        }
        // T_IJ = -T_II W (W through this wave's scratch; LDS is in order per wave)
#pragma unroll
        for (int i = 0; i < 4; ++i) wsc[(4 * g4 + i) * 17 + l16] = w[i];
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int k = 4 * ks + g4;
          float av = Ti[(16 * I + l16) * LP + 16 * I + k];
          if (up ? k < l16 : k > l16) av = 0.f;
          t = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wsc[k * 17 + l16], t, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Ti[(16 * I + 4 * g4 + i) * LP + 16 * J + l16] = -t[i];
      }
    };
    if constexpr (NB == 4) {
      if (wave == 0) {
        if (fwd_on) column(0, 0);
      } else if (wave == 1) {
        if (rev_on) column(1, 3);
      } else if (wave == 2) {
        if (fwd_on) { column(0, 1); column(0, 2); }
      } else {
        if (rev_on) { column(1, 2); column(1, 1); }
      }
    } else {
      if (wave == 0 && fwd_on) column(0, 0);
      if (wave == 1 && rev_on) column(1, 1);
    }
  }
  __syncthreads();

  // ---- both triangles to the workspace, 16 bytes per store ----
  {
    constexpr int EPS = 16 / (int)sizeof(MT);
    MT* tri = static_cast<MT*>(a.tri) + cid * C * C;
    MT* pqk = static_cast<MT*>(a.pqk) + cid * C * C;
    for (int p = tid; p < C * C / EPS; p += 256) {
      const int r = (p * EPS) / C, c0 = (p * EPS) % C;
      MT tv[EPS], pv[EPS];
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int col = c0 + e;
        const bool keep = (col < r && fwd_on) || (col > r && rev_on);
        tv[e] = (MT)(keep ? Ti[r * LP + col] : 0.f);
        pv[e] = (keep || col == r) ? Pst[r * PP + col] : (MT)0.f;
      }
      __builtin_memcpy(tri + p * EPS, tv, 16);
      __builtin_memcpy(pqk + p * EPS, pv, 16);
    }
  }
  // ---- per-token scales and the chunk decay ----
  if (tid < C) {
    const bool in = (t0 + tid) < T;
    const float rk = s_rk[tid], rq = s_rq[tid];
    if (fwd_on) {
      const float g = s_g[0][tid], gl = s_g[0][C - 1];
      const float eg = exp2f(g);
      float4 v = in ? make_float4(s_bt[0][tid], eg * rk, eg * rq, exp2f(gl - g) * rk) : make_float4(0.f, 0.f, 0.f, 0.f);
      a.sc[(fslot * nch + cid) * C + tid] = v;
      if (tid < 4) a.pdg[((size_t)fslot * nch + cid) * (C + 4) + C + tid] = tid == 0 ? exp2f(gl) : 0.f;
    }
    if (rev_on) {
      const float g = s_g[1][tid], gl = s_g[1][0];
      const float eg = exp2f(g);
      float4 v = in ? make_float4(s_bt[1][tid], eg * rk, eg * rq, exp2f(gl - g) * rk) : make_float4(0.f, 0.f, 0.f, 0.f);
      a.sc[(rslot * nch + cid) * C + tid] = v;
      if (tid < 4) a.pdg[((size_t)rslot * nch + cid) * (C + 4) + C + tid] = tid == 0 ? exp2f(gl) : 0.f;
    }
  }

  // ---- bidirectional scans: the second visitor of a chunk in the state
  // chain recognises the first visitor's readout by this all-ones NaN fill
  // ("not written yet"; arithmetic never produces it).  Last, so these stores
  // never queue ahead of the loads above. ----
  if (a.zero_out) {
    const int dv4 = a.dv / 4;
    const float fill = __uint_as_float(0xFFFFFFFFu);
    for (int p = tid; p < C * dv4; p += 256) {
      const int row = p / dv4, cp = (p % dv4) * 4;
      const int64_t t = t0 + row;
      if (t < T) *reinterpret_cast<f32x4*>(a.out + ((b * T + t) * H + h) * a.dv + cp) = f32x4{fill, fill, fill, fill};
    }
  }
}

template <typename MT, int DK, int C>
hipError_t launch_prep(const ScanArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.NC, (unsigned)(a.B * a.H));
  hipLaunchKernelGGL((chunk_prep_kernel<MT, DK, C>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

#define GDN_INST_PREP(MT, DK, C) template hipError_t launch_prep<MT, DK, C>(const ScanArgs&, hipStream_t);
GDN_INST_PREP(float, 64, 32)
GDN_INST_PREP(float, 64, 64)
GDN_INST_PREP(float, 128, 32)
GDN_INST_PREP(float, 128, 64)
GDN_INST_PREP(bf16, 64, 32)
GDN_INST_PREP(bf16, 64, 64)
GDN_INST_PREP(bf16, 128, 32)
GDN_INST_PREP(bf16, 128, 64)

}  // namespace gdn

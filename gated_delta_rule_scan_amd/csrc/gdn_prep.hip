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
  __shared__ __align__(16) float s_rk[C], s_rq[C], s_qk[C];  // row scales, raw q.k of each token
  __shared__ __align__(16) float s_raw[4][64], s_g[2][C];  // raw gates as loaded (see below); cumulative log2-gates

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
  // Workgroups are numbered in the order the state chain consumes the
  // chunks (a bidirectional scan takes both ends first), and each (batch,
  // head) sequence's chunks go to the XCD its state-chain workgroups run on
  // (consecutive ids are dealt round-robin over the eight XCDs).
  const int nbh = (int)(a.B * a.H), G = (nbh + 7) / 8;
  const int id = blockIdx.x;
  const int64_t bh = (int64_t)((id >> 3) % G) * 8 + (id & 7);
  const int order = (id >> 3) / G;  // position in the consumption order
  const int NCi = (int)a.NC;
  int64_t c;
  if (a.fwd_on && a.rev_on) {
    const int J = (NCi + 1) / 2;  // even positions take chunks [0, J), odd ones [J, NC) from the end
    const int j = order >> 1;
    if ((order & 1) && j >= NCi - J) return;
    c = (order & 1) ? NCi - 1 - j : j;
  } else {
    c = a.rev_on ? NCi - 1 - order : order;
  }
  if (bh >= nbh) return;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t T = a.T, H = a.H, B = a.B;
  const int64_t t0 = c * C;
  const int64_t cid = bh * a.NC + c;
  const int fwd_on = a.fwd_on, rev_on = a.rev_on;
  const int fslot = 0, rslot = fwd_on ? 1 : 0;
  const size_t nch = (size_t)a.B * a.H * a.NC;
  const int nrows = (int)(T - t0 < C ? T - t0 : C);  // valid tokens of this chunk (>= 1)
  constexpr float kLog2e = 1.4426950408889634f;

  // ---- every global read of the kernel, issued at once ----
  // Raw q and k rows (16-byte pieces; rows past the sequence read as zero),
  // and one gate per lane: wave 0 the forward log-gates in token order, wave 1
  // the reverse log-gates in reverse token order (the reverse visiting
  // order), waves 2 and 3 the forward and reverse write strengths.
  constexpr int PR = DK / EP;    // pieces per row
  constexpr int RPI = 256 / PR;  // rows per pass of the workgroup
  constexpr int NPT = C / RPI;   // pieces per thread and matrix
  static_assert(256 % PR == 0 && C % RPI == 0, "piece split");
  const int prow = tid / PR, pcol = (tid % PR) * EP;
  const uint32_t rowb = (uint32_t)(H * DK * (int64_t)sizeof(MT));
  const size_t kq0 = (size_t)((b * T + t0) * H + h) * DK;
  const uint32_t kq_ext = (uint32_t)(nrows - 1) * rowb + DK * (uint32_t)sizeof(MT);
  const rsrc_t rq = make_rsrc(static_cast<const MT*>(a.q) + kq0, kq_ext);
  const rsrc_t rk = make_rsrc(static_cast<const MT*>(a.k) + kq0, kq_ext);
  f32x4 vq[NPT], vk[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const uint32_t off = (uint32_t)(prow + RPI * i) * rowb + pcol * (uint32_t)sizeof(MT);
    vq[i] = bload16(rq, off);
    vk[i] = bload16(rk, off);
  }
  float gate;
  {
    const int dir = wave & 1;                   // waves 0, 2: forward; 1, 3: reverse
    const bool on = dir == 0 ? fwd_on : rev_on;
    const int slot = dir == 0 ? fslot : rslot;
    const float* src = wave < 2 ? a.log_alpha : a.beta;
    const rsrc_t rg = make_rsrc(src + ((slot * B + b) * T + t0) * H + h, on ? (uint32_t)((nrows - 1) * H + 1) * 4u : 0u);
    const int tok = wave == 1 ? C - 1 - lane : lane;
    gate = bload4(rg, lane < C ? (uint32_t)(tok * H) * 4u : 0xFFFFFFF0u);
  }

  // ---- row scales from the registers, operands into LDS ----
  {
    auto elem = [](const f32x4& v, int e) -> float {  // element e of a 16-byte piece
      if constexpr (sizeof(MT) == 2) {
        return (float)__builtin_bit_cast(bf16x8, v)[e];
      } else {
        return v[e];
      }
    };
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      float sq = 0.f, sk = 0.f, sqk = 0.f;
      if constexpr (sizeof(MT) == 2) {
        // two bf16 products per instruction (exact in fp32), fp32 sums; the
        // pairs come from one bit cast of the whole piece and vector shuffles
        const bf16x8 q8 = __builtin_bit_cast(bf16x8, vq[i]), k8 = __builtin_bit_cast(bf16x8, vk[i]);
#define GDN_DOT2_PAIR(a, b)                                                                   \
  {                                                                                           \
    const auto xq = __builtin_shufflevector(q8, q8, a, b);                                    \
    const auto xk = __builtin_shufflevector(k8, k8, a, b);                                    \
    sq = __builtin_amdgcn_fdot2_f32_bf16(xq, xq, sq, false);                                  \
    sk = __builtin_amdgcn_fdot2_f32_bf16(xk, xk, sk, false);                                  \
    sqk = __builtin_amdgcn_fdot2_f32_bf16(xq, xk, sqk, false);                                \
  }
        GDN_DOT2_PAIR(0, 1) GDN_DOT2_PAIR(2, 3) GDN_DOT2_PAIR(4, 5) GDN_DOT2_PAIR(6, 7)
#undef GDN_DOT2_PAIR
      } else {
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          const float xq = elem(vq[i], e), xk = elem(vk[i], e);
          sq = fmaf(xq, xq, sq);
          sk = fmaf(xk, xk, sk);
          sqk = fmaf(xq, xk, sqk);
        }
      }
#pragma unroll
      for (int m = 1; m < PR; m <<= 1) {
        sq += __shfl_xor(sq, m, 64);
        sk += __shfl_xor(sk, m, 64);
        sqk += __shfl_xor(sqk, m, 64);
      }
      const int row = prow + RPI * i;
      if (tid % PR == 0) {
        s_rq[row] = 1.0f / fmaxf(sqrtf(sq), kNormEps);
        s_rk[row] = 1.0f / fmaxf(sqrtf(sk), kNormEps);
        s_qk[row] = sqk;
      }
      *reinterpret_cast<f32x4*>(Qs + row * KP + pcol) = vq[i];
      *reinterpret_cast<f32x4*>(Ks + row * KP + pcol) = vk[i];
    }
  }
  // every wave parks its gate in LDS at once (so no path leaves the load
  // pending); rows 2 and 3 are the write strengths in token order
  s_raw[wave][lane] = gate;
  const float (*s_bt)[64] = s_raw + 2;

  // ---- bidirectional scans: the second visitor of a chunk in the state
  // chain recognises the first visitor's readout by this all-ones NaN fill
  // ("not written yet"; arithmetic never produces it).  Issued after every
  // read of the kernel has returned, so it never delays them. ----
  if (a.zero_out) {
    const int sh = 29 - __builtin_clz((unsigned)a.dv);  // log2(dv / 4): 16-byte pieces per row (a power of two)
    const uint32_t orow = (uint32_t)(H * a.dv) * 4u;
    const rsrc_t ro = make_rsrc(a.out + ((b * T + t0) * H + h) * a.dv, (uint32_t)(nrows - 1) * orow + (uint32_t)a.dv * 4u);
    const float fn = __uint_as_float(0xFFFFFFFFu);
    const f32x4 fill = f32x4{fn, fn, fn, fn};
    for (int p = tid; p < (C << sh); p += 256)
      bstore16_agent(ro, (uint32_t)(p >> sh) * orow + (uint32_t)(p & ((1 << sh) - 1)) * 16u, fill);
  }
  __syncthreads();

  // chunk-local cumulative log-gates in log2 units (every decay factor below
  // is one exp2 of a difference): wave 0 the inclusive prefix sums in token
  // order, wave 1 the inclusive suffix sums, each as a wave-wide scan; read
  // only after the next barrier
  if (wave < 2) {
    float s = s_raw[wave][lane];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float o = __shfl_up(s, d, 64);
      if (lane >= d) s += o;
    }
    if (lane < C) s_g[wave][wave == 0 ? lane : C - 1 - lane] = s * kLog2e;
  }

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
  // (the erase-free variant has no erase term: L = 0, so (I + L)^{-1} = I)
  const float erase_w = a.erase ? 1.f : 0.f;
  // Lane (l16, g4) of tile (ti, tj) holds column 16 tj + l16 of rows
  // 16 ti + 4 g4 + i.  Below the diagonal the forward direction's entries,
  // above it the reverse direction's; the diagonal (the self terms) is
  // written beside the diagonal solve below.
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = wave + 4 * j;
    if (u < NT2) {
      const int ti = u / NB, tj = u % NB;
      const int col = 16 * tj + l16, r0 = 16 * ti + 4 * g4;
      const float gfc = s_g[0][col], grc = s_g[1][col], rkc = s_rk[col];
      const f32x4 gf = *reinterpret_cast<const f32x4*>(&s_g[0][r0]);
      const f32x4 gr = *reinterpret_cast<const f32x4*>(&s_g[1][r0]);
      const f32x4 bf = *reinterpret_cast<const f32x4*>(&s_bt[0][r0]);
      const f32x4 br = *reinterpret_cast<const f32x4*>(&s_bt[1][r0]);
      const f32x4 rkr = *reinterpret_cast<const f32x4*>(&s_rk[r0]);
      const f32x4 rqr = *reinterpret_cast<const f32x4*>(&s_rq[r0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        // 0/1 weights of the two directions (arithmetic selects: no branches)
        const float wf = (col < r && fwd_on) ? 1.f : 0.f, wr = (col > r && rev_on) ? 1.f : 0.f;
        // decay between the two tokens (<= 0 in log2 units; zero where
        // unused, so it never overflows); below 2^-126 it may flush to zero
        const float gd = fmaf(wf, gf[i] - gfc, wr * (gr[i] - grc));
        const float e = __builtin_amdgcn_exp2f(gd);
        const float lm = e * fmaf(wf, bf[i], wr * br[i]) * erase_w;
        const float pm = e * (wf + wr);
        Lm[r * LP + col] = (rkr[i] * rkc) * accG[j][i] * lm;
        Pst[r * PP + col] = (MT)((rqr[i] * rkc) * accP[j][i] * pm);
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
    // The column is written out only at the end, so every read of L can be
    // issued ahead of the chain.  One instance per direction keeps every
    // index a compile-time constant (the running sums stay in registers).
    auto solve = [&](auto rev_tag) {
      constexpr bool R = decltype(rev_tag)::value;
      float acc[16], x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int i = R ? 15 - ii : ii;  // visiting order
        const bool after = R ? (i < jc) : (i > jc);
        x[i] = i == jc ? 1.f : (after ? -acc[i] : 0.f);
#pragma unroll
        for (int rr = ii + 1; rr < 16; ++rr) {
          const int r = R ? 15 - rr : rr;
          acc[r] = fmaf(Lm[(b0 + r) * LP + b0 + i], x[i], acc[r]);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (R ? i <= jc : i >= jc) Ti[(b0 + i) * LP + b0 + jc] = x[i];
    };
    if (dir == 0 && fwd_on) solve(std::false_type{});
    if (dir == 1 && rev_on) solve(std::true_type{});
  } else if (tid - 2 * NB * 16 < 2 * C) {
    // ---- meanwhile, per-token scales and the chunk decays ----
    const int idx = tid - 2 * NB * 16;
    const int dir = idx / C, tok = idx % C;
    // self term q^_t . k^_t: the operand type's rounding on the diagonal of
    // the decayed q.k tile, the part it drops into each direction's record
    const float rk = s_rk[tok], rq = s_rq[tok];
    const float self = rq * rk * s_qk[tok];
    const MT self_mt = (MT)self;
    if (dir == 0) Pst[tok * PP + tok] = self_mt;
    if (dir == 0 ? fwd_on : rev_on) {
      const int slot = dir == 0 ? fslot : rslot;
      const bool in = tok < nrows;
      const float g = s_g[dir][tok], gl = s_g[dir][dir == 0 ? C - 1 : 0];
      const float eg = exp2f(g);
      const rsrc_t rs = make_rsrc(a.sc + (slot * nch + cid) * C, C * 16);
      // {beta, e^g rk (erase term of the pseudo-values; 0 without it), e^g rq, e^(gn-g) rk}
      bstore16_agent(rs, tok * 16,
                     in ? f32x4{s_bt[dir][tok], a.erase ? eg * rk : 0.f, eg * rq, exp2f(gl - g) * rk} : f32x4{0.f, 0.f, 0.f, 0.f});
      const rsrc_t rp = make_rsrc(a.pdg + ((size_t)slot * nch + cid) * pdg_stride(C), (C + 4) * 4);
      bstore4_agent(rp, tok * 4, self - (float)self_mt);
      if (tok < 4) bstore4_agent(rp, (C + tok) * 4, tok == 0 ? exp2f(gl) : 0.f);
    }
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
    const rsrc_t rt = make_rsrc(static_cast<MT*>(a.tri) + cid * C * C, C * C * (int)sizeof(MT));
    const rsrc_t rp = make_rsrc(static_cast<MT*>(a.pqk) + cid * C * C, C * C * (int)sizeof(MT));
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
      f32x4 t16, p16;
      __builtin_memcpy(&t16, tv, 16);
      __builtin_memcpy(&p16, pv, 16);
      bstore16_agent(rt, p * 16, t16);
      bstore16_agent(rp, p * 16, p16);
    }
  }

  // ---- publish: every store above is agent-scope (written through this
  // XCD's L2: the state chain may run on another XCD, whose L2 misses on
  // these lines -- none of them is read before the flag, and no cache line
  // holds two chunks' data).  Once each wave's stores have drained, the
  // chunk's ready flag ----
  if (a.ready) {
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.ready + cid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__global__ __launch_bounds__(256) void clear_ready_kernel(unsigned* ready, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) ready[i] = 1u;  // pending
}

hipError_t launch_clear_ready(unsigned* ready, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(clear_ready_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, ready, n);
  return hipGetLastError();
}

template <typename MT, int DK, int C>
hipError_t launch_prep(const ScanArgs& a, hipStream_t stream, hipFuncAttributes* query) {
  if (query) return hipFuncGetAttributes(query, reinterpret_cast<const void*>(&chunk_prep_kernel<MT, DK, C>));
  const int64_t G = (a.B * a.H + 7) / 8;
  const int64_t slots = (a.fwd_on && a.rev_on) ? 2 * ((a.NC + 1) / 2) : a.NC;
  hipLaunchKernelGGL((chunk_prep_kernel<MT, DK, C>), dim3((unsigned)(slots * G * 8)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

#define GDN_INST_PREP(MT, DK, C) \
  template hipError_t launch_prep<MT, DK, C>(const ScanArgs&, hipStream_t, hipFuncAttributes*);
GDN_INST_PREP(float, 64, 32)
GDN_INST_PREP(float, 64, 64)
GDN_INST_PREP(float, 128, 32)
GDN_INST_PREP(float, 128, 64)
GDN_INST_PREP(bf16, 64, 32)
GDN_INST_PREP(bf16, 64, 64)
GDN_INST_PREP(bf16, 128, 32)
GDN_INST_PREP(bf16, 128, 64)

}  // namespace gdn

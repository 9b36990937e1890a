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

// x plus its value in another lane of the same 16-lane row, moved by a data
// parallel primitive (no LDS): 0xB1 and 0x4E swap neighbouring lanes and
// lane pairs of each quad, 0x141 mirrors each half row, 0x140 each row
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over each aligned group of N consecutive lanes (N a power of two, 2 ..
// 64), the same in every lane of the group: within a row by permutations,
// across rows by lane shuffles
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "group size");
  x = dpp_add<0xB1>(x);
  if constexpr (N >= 4) x = dpp_add<0x4E>(x);
  if constexpr (N >= 8) x = dpp_add<0x141>(x);
  if constexpr (N >= 16) x = dpp_add<0x140>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// v from another lane (DPP control CTRL, rows in the mask ROWS; 0 where no
// lane is read), a double moved as its two halves
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROWS, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROWS, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// lanes within each row of 16, then the last lane of row 0 (2) added to row 1
// (3), then the last lane of row 1 added to rows 2 and 3
__device__ __forceinline__ double wave_prefix_sum(double x) {
  x += dpp_f64<0x111, 0xF>(x);
  x += dpp_f64<0x112, 0xF>(x);
  x += dpp_f64<0x114, 0xF>(x);
  x += dpp_f64<0x118, 0xF>(x);
  x += dpp_f64<0x142, 0xA>(x);
  x += dpp_f64<0x143, 0xC>(x);
  return x;
}

template <typename MT, int DK, int C>
struct PrepSmem {
  static constexpr int EP = 16 / (int)sizeof(MT);       // elements per 16-byte piece
  static constexpr int KP = DK + EP;                    // padded row pitch of staged q/k
  static constexpr int NB = C / 16;                     // 16 x 16 blocks per side
  // The inverse works on fp32 16 x 16 blocks, each stored as the register
  // image of the matrix-core operand that reads it (fragment order below),
  // so that a fragment read or a result write is one consecutive dword per
  // lane, free of LDS bank conflicts:
  //   * L's off-diagonal blocks in A order: entry (r, c) at 64 (c % 4) + 16 (c / 4) + r;
  //   * the inverse's blocks in B order: entry (r, c) at 64 (r % 4) + 16 (r / 4) + c,
  //     which is also where a 16 x 16 product leaves entry (r, c); block
  //     stride 272 (16 dwords of padding), so the four diagonal blocks,
  //     written column by column by the substitution, start in different banks;
  //   * L's diagonal blocks transposed for the substitution: rows of 20, blocks
  //     of 336 dwords (the same bank spreading for their 16-byte reads).
  static constexpr int LB = 256, TB = 272, DR = 20, DB = 336;
  static constexpr int LM_F = NB * (NB - 1) * LB, TI_F = NB * NB * TB, LD_F = NB * DB;
  static constexpr size_t kq_bytes = (size_t)2 * C * KP * sizeof(MT);
  static constexpr size_t inv_bytes = (size_t)(LM_F + TI_F + LD_F) * 4;
  static constexpr size_t region = kq_bytes > inv_bytes ? kq_bytes : inv_bytes;
};

// PLO: the low parts of the decayed q.k tile are written too (exclusive
// readouts on bf16 operands).  Without them, bf16 operands fit four
// workgroups per compute unit (40 KB of LDS each) when the registers do too.
template <typename MT, int DK, int C, bool PLO>
__global__ __launch_bounds__(256, (PLO || sizeof(MT) == 4) ? 2 : 4) void chunk_prep_kernel(ScanArgs a) {
  using SM = PrepSmem<MT, DK, C>;
  using M = Mma<MT>;
  constexpr int EP = SM::EP, KP = SM::KP, NB = SM::NB;
  constexpr int TB = SM::TB, DR = SM::DR, DB = SM::DB;

  __shared__ __align__(16) unsigned char smem[SM::region];
  __shared__ __align__(16) float s_rk[C], s_rq[C], s_qk[C];  // row scales, raw q.k of each token
  __shared__ __align__(16) float s_raw[4][64];  // raw gates as loaded (see below)
  __shared__ __align__(16) double s_g[2][C];   // cumulative log2-gates (double: see the scan)

  MT* Ks = reinterpret_cast<MT*>(smem);
  MT* Qs = Ks + C * KP;
  // after the Gram products, the q/k staging area holds the inverse's blocks
  float* Lm = reinterpret_cast<float*>(smem);  // L's off-diagonal blocks, A order
  float* Ti = Lm + SM::LM_F;                   // the inverse's blocks, B order
  // the diagonal 16 x 16 blocks of L transposed (the forward entries below
  // the diagonal, the reverse ones above), read by the diagonal solve
  float* Ld = Ti + SM::TI_F;
  // block (I, K) of L (I != K) and block (R, Q) of the inverse
  auto lblk = [&](int I, int K) { return Lm + (I * (NB - 1) + (K < I ? K : K - 1)) * SM::LB; };
  auto tblk = [&](int R, int Q) { return Ti + (R * NB + Q) * TB; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  // Workgroups are numbered in the order the state chain consumes the
  // chunks (a bidirectional scan takes both ends first); consecutive ids are
  // dealt round-robin over the eight XCDs.  Run before the chain, all heads of
  // one (batch, chunk) go to one XCD: a 128-byte line of gates ([dirs, B, T,
  // H] layout) holds every head of a few tokens, so the line is fetched into
  // that XCD's L2 once (dealt by sequence, every XCD fetched every gate line:
  // eight times the gates' bytes, 0.12 of the 0.55 GB the pass reads at the
  // 480p bidirectional shape).  Run beside the chain, each sequence's chunks
  // go to the XCD its state-chain workgroups run on.
  const int nbh = (int)(a.B * a.H), G = (nbh + 7) / 8;
  const int id = blockIdx.x;
  const int NCi = (int)a.NC;
  int64_t bh;
  int order;  // position in the consumption order
  if (a.ready) {
    bh = (int64_t)((id >> 3) % G) * 8 + (id & 7);
    order = (id >> 3) / G;
  } else {
    const int Hi = (int)a.H, Bi = (int)a.B, p = id >> 3;
    const int gi = (p / Hi) * 8 + (id & 7);  // (position, batch) group
    order = gi / Bi;
    bh = (int64_t)(gi % Bi) * Hi + p % Hi;
  }
  if (order >= ((a.fwd_on && a.rev_on) ? 2 * ((NCi + 1) / 2) : NCi)) return;
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
  constexpr double kLog2eD = 1.4426950408889634;
  const bool ag = ws_agent_stores<C>(a);  // workspace stores at agent scope (see there)

  // ---- every global read of the kernel, issued at once ----
  // Raw q and k rows (16-byte pieces; rows past the sequence read as zero),
  // and one gate per lane: wave 0 the forward log-gates in token order, wave 1
  // the reverse log-gates in reverse token order (the reverse visiting
  // order), waves 2 and 3 the forward and reverse write strengths.
  constexpr int PR = DK / EP;    // pieces per row
  constexpr int RPI = 256 / PR;  // rows per pass of the workgroup
  constexpr int NPT = (C + RPI - 1) / RPI;  // pieces per thread and matrix
  static_assert(256 % PR == 0 && (C % RPI == 0 || NPT == 1), "piece split");
  // a 16-token chunk with 64-wide bf16 rows: a pass covers 32 rows, and the
  // lanes of rows 16..31 take part in the row sums but store nothing
  constexpr bool ROWS_PAST = C % RPI != 0;
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
      sq = group_sum<PR>(sq);
      sk = group_sum<PR>(sk);
      sqk = group_sum<PR>(sqk);
      const int row = prow + RPI * i;
      if (ROWS_PAST && row >= C) continue;
      if (tid % PR == 0) {
        // 1 / max(|x|, eps) as a reciprocal square root (one rounding more
        // than a divide: relative error ~1e-7)
        constexpr float e2 = kNormEps * kNormEps;
        s_rq[row] = sq > e2 ? __builtin_amdgcn_rsqf(sq) : 1.0f / kNormEps;
        s_rk[row] = sk > e2 ? __builtin_amdgcn_rsqf(sk) : 1.0f / kNormEps;
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
  // chain must know when the first visitor's readout is in `out`.  bf16
  // operands: the chunk's combine flags, cleared here (the state chain
  // starts only after this kernel has finished).  fp32 operands: `out` is
  // filled with the all-ones NaN ("not written yet"; first visitors store
  // canonical NaNs, so a readout never carries it), issued after every read
  // of the kernel has returned, so it never delays them. ----
  if (a.part_flags) {
    const int nfl = a.dv >> 4;
    if (tid < nfl) a.part_flags[cid * nfl + tid] = 0u;
  }
  if (a.zero_out) {
    const int sh = 29 - __builtin_clz((unsigned)a.dv);  // log2(dv / 4): 16-byte pieces per row (a power of two)
    const uint32_t orow = (uint32_t)(H * a.dv) * 4u;
    const rsrc_t ro = make_rsrc(a.out + ((b * T + t0) * H + h) * a.dv, (uint32_t)(nrows - 1) * orow + (uint32_t)a.dv * 4u);
    const float fn = __uint_as_float(0xFFFFFFFFu);
    const f32x4 fill = f32x4{fn, fn, fn, fn};
    for (int p = tid; p < (C << sh); p += 256)
      bstore16_ws(ag, ro, (uint32_t)(p >> sh) * orow + (uint32_t)(p & ((1 << sh) - 1)) * 16u, fill);
  }
  __syncthreads();

  // chunk-local cumulative log-gates in log2 units (every decay factor below
  // is one exp2 of a difference): wave 0 the inclusive prefix sums in token
  // order, wave 1 the inclusive suffix sums, each as a wave-wide scan; read
  // only after the next barrier.  The sums run in double: over a chunk they
  // reach hundreds (fast decay), where one fp32 rounding is already a
  // relative error of 1e-5 in every decay factor taken as a difference of
  // two of them; in double, each difference is rounded once, to fp32.
  if (wave < 2) {
    const double s = wave_prefix_sum((double)s_raw[wave][lane] * kLog2eD);
    if (lane < C) s_g[wave][wave == 0 ? lane : C - 1 - lane] = s;
  }

  // ---- Gram K K^T and Q K^T on the matrix cores (raw operands, fp32
  // accumulate), taken transposed: lane (l16, g4) of tile (ti, tj) ends up
  // with row 16 ti + l16 and columns 16 tj + 4 g4 + i (i = 0..3), four
  // consecutive entries of one row, as the decayed q.k tile is stored ----
  constexpr int NT2 = NB * NB;
  constexpr int UPW = (NT2 + 3) / 4;
  f32x4 accG[UPW], accP[UPW];
  // with four block columns a wave's tiles share their column block (tj =
  // wave): its k fragments are read once
  typename M::frag kcw[DK / 32];
  if constexpr (NB == 4) {
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) kcw[ks] = M::load(Ks + (16 * wave + l16) * KP + 32 * ks + 8 * g4);
  }
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    accG[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    accP[j] = accG[j];
    const int u = wave + 4 * j;
    if (u < NT2) {
      const int ti = u / NB, tj = u % NB;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const typename M::frag kr = M::load(Ks + (16 * ti + l16) * KP + 32 * ks + 8 * g4);
        const typename M::frag qr = M::load(Qs + (16 * ti + l16) * KP + 32 * ks + 8 * g4);
        const typename M::frag kc = NB == 4 ? kcw[ks] : M::load(Ks + (16 * tj + l16) * KP + 32 * ks + 8 * g4);
        accG[j] = M::mma(kc, kr, accG[j]);
        accP[j] = M::mma(kc, qr, accP[j]);
      }
    }
  }
  __syncthreads();  // q/k staging area is reused below

  // ---- gated, scaled triangles: L into LDS, the decayed Q^K^^T (with the
  // self terms on its diagonal) straight to the workspace ----
  // (the erase-free variant has no erase term: L = 0, so (I + L)^{-1} = I)
  // Below the diagonal the forward direction's entries, above it the
  // reverse direction's; entries of a direction that is off are zero.  With
  // PLO, the part of each decayed q.k entry that bf16 drops goes to its own
  // tile (zero on the diagonal, whose remainder is in the chunk record).
  const float erase_w = a.erase ? 1.f : 0.f;
  {
    const rsrc_t rpq = make_rsrc(static_cast<MT*>(a.pqk) + cid * C * C, C * C * (int)sizeof(MT));
    const rsrc_t rpl = PLO ? make_rsrc(static_cast<MT*>(a.pq_lo) + cid * C * C, C * C * (int)sizeof(MT)) : rpq;
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = wave + 4 * j;
      if (u >= NT2) continue;
      const int ti = u / NB, tj = u % NB;
      const int r = 16 * ti + l16, c0 = 16 * tj + 4 * g4;
      const float rkr = s_rk[r], rqr = s_rq[r];
      const f32x4 rkc = *reinterpret_cast<const f32x4*>(&s_rk[c0]);
      float pv[4] = {0.f, 0.f, 0.f, 0.f};
      if (ti != tj) {
        // a tile off the diagonal holds one direction's entries; the other
        // direction never reads it
        const int dir = ti > tj ? 0 : 1;
        if (dir == 0 ? fwd_on : rev_on) {
          const double gr = s_g[dir][r];
          const float fl = rkr * s_bt[dir][r] * erase_w;  // the row's factor of L
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = c0 + i;
            // decay between the two tokens (<= 0 in log2 units; below
            // 2^-126 it may flush to zero) times the column's k scale
            const float ek = __builtin_amdgcn_exp2f((float)(gr - s_g[dir][c])) * rkc[i];
            // entry (l16, 4 g4 + i) of block (ti, tj), A order
            lblk(ti, tj)[64 * i + lane] = (fl * ek) * accG[j][i];
            pv[i] = (rqr * ek) * accP[j][i];
          }
        }
      } else {
        const double grf = s_g[0][r], grr = s_g[1][r];
        const float flf = rkr * s_bt[0][r] * erase_w, flr = rkr * s_bt[1][r] * erase_w;
        // the self term q^_t . k^_t (its remainder: the chunk record)
        const float self = rqr * rkr * s_qk[r];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = c0 + i;
          // an entry is the reverse direction's above the diagonal, the
          // forward one's below (selects, no branches); unused entries take a
          // zero exponent, so they never overflow, and a zero factor
          const bool up = c > r;
          const uint32_t on = (up ? rev_on != 0 : (c < r && fwd_on)) ? ~0u : 0u;
          // both directions' sums are read and one is kept (a read under the
          // condition would become a branch and an LDS round trip per entry)
          const double g0c = s_g[0][c], g1c = s_g[1][c];
          const float gd = __uint_as_float(__float_as_uint((float)((up ? grr : grf) - (up ? g1c : g0c))) & on);
          const float ek = __builtin_amdgcn_exp2f(gd) * __uint_as_float(__float_as_uint(rkc[i]) & on);
          Ld[tj * DB + (4 * g4 + i) * DR + l16] = ((up ? flr : flf) * ek) * accG[j][i];  // the block transposed
          pv[i] = c == r ? self : (rqr * ek) * accP[j][i];
        }
      }
      const uint32_t off = (uint32_t)(r * C + c0) * (uint32_t)sizeof(MT);
      if constexpr (sizeof(MT) == 2) {
        bf16x4 ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ph[i] = (bf16)pv[i];
          pl[i] = (c0 + i == r) ? (bf16)0.f : (bf16)(pv[i] - (float)ph[i]);
        }
        uint32_t w[2], wl[2];
        __builtin_memcpy(w, &ph, 8);
        __builtin_memcpy(wl, &pl, 8);
        bstore8_ws(ag, rpq, off, w[0], w[1]);
        if constexpr (PLO) bstore8_ws(ag, rpl, off, wl[0], wl[1]);
      } else {
        bstore16_ws(ag, rpq, off, f32x4{pv[0], pv[1], pv[2], pv[3]});
      }
    }
  }
  __syncthreads();

  // ---- diagonal 16 x 16 blocks: one column of the inverse per thread ----
  if (tid < 2 * NB * 16) {
    // with 64-token chunks each direction is one wave (uniform operands)
    const int dir = NB == 4 ? (wave & 1) : tid / (NB * 16);
    const int blk = (tid / 16) % NB;
    const int jc = tid % 16;
    // column jc of (I + L_bb)^{-1} by forward substitution in visiting
    // order, column-oriented: once x_i is known it is folded into every
    // later row's running sum, so the dependent chain is 16 steps long.
    // Column i of L_bb is row i of the transposed copy, read four rows at a
    // time; the column is written out only at the end, so every read of L
    // can be issued ahead of the chain.  One instance per direction keeps
    // every index a compile-time constant (the running sums stay in
    // registers).
    const float* ldb = Ld + blk * DB;
    auto solve = [&](auto rev_tag) {
      constexpr bool R = decltype(rev_tag)::value;
      // the rows of group m (4 m .. 4 m + 3) that come after i
      auto live = [](int i, int m) { return R ? 4 * m < i : 4 * m + 3 > i; };
      float acc[16], x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      // column i of L_bb, read one step ahead (a step is one scheduling
      // region, so the reads are not all hoisted to the start)
      f32x4 cur[4], nxt[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i0 = R ? 15 : 0;
        cur[m] = live(i0, m) ? *reinterpret_cast<const f32x4*>(ldb + i0 * DR + 4 * m) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int i = R ? 15 - ii : ii;  // visiting order
        if (ii < 15) {
          const int in = R ? i - 1 : i + 1;
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (live(in, m)) nxt[m] = *reinterpret_cast<const f32x4*>(ldb + in * DR + 4 * m);
        }
        const bool after = R ? (i < jc) : (i > jc);
        x[i] = i == jc ? 1.f : (after ? -acc[i] : 0.f);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (!live(i, m)) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * m + e;
            if (R ? r < i : r > i) acc[r] = fmaf(cur[m][e], x[i], acc[r]);
          }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) cur[m] = nxt[m];
        // the step's products stay in the step (not sunk to their uses,
        // which would keep every read of L live at once)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (R ? r < i : r > i) asm volatile("" : "+v"(acc[r]));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (R ? i <= jc : i >= jc) tblk(blk, blk)[64 * (i & 3) + 16 * (i >> 2) + jc] = x[i];
    };
    if (dir == 0 && fwd_on) solve(std::false_type{});
    if (dir == 1 && rev_on) solve(std::true_type{});
  } else if (tid - 2 * NB * 16 < 2 * C) {
    // ---- meanwhile, per-token scales and the chunk decays ----
    const int idx = tid - 2 * NB * 16;
    const int dir = NB == 4 ? (wave & 1) : idx / C, tok = idx % C;
    // self term q^_t . k^_t: the operand type's rounding on the diagonal of
    // the decayed q.k tile, the part it drops into each direction's record
    const float rk = s_rk[tok], rq = s_rq[tok];
    const float self = rq * rk * s_qk[tok];
    const MT self_mt = (MT)self;
    if (dir == 0 ? fwd_on : rev_on) {
      const int slot = dir == 0 ? fslot : rslot;
      const bool in = tok < nrows;
      const double g = s_g[dir][tok], gl = s_g[dir][dir == 0 ? C - 1 : 0];
      const float eg = exp2f((float)g);
      const rsrc_t rs = make_rsrc(a.sc + (slot * nch + cid) * C, C * 16);
      // {beta, e^g rk (erase term of the pseudo-values; 0 without it), e^g rq, e^(gn-g) rk}
      bstore16_ws(ag, rs, tok * 16,
                     in ? f32x4{s_bt[dir][tok], a.erase ? eg * rk : 0.f, eg * rq, exp2f((float)(gl - g)) * rk}
                        : f32x4{0.f, 0.f, 0.f, 0.f});
      const rsrc_t rp = make_rsrc(a.pdg + ((size_t)slot * nch + cid) * pdg_stride(C), (C + 4) * 4);
      bstore4_ws(ag, rp, (4 + tok) * 4, self - (float)self_mt);
      if (tok < 4) bstore4_ws(ag, rp, tok * 4, tok == 0 ? exp2f((float)gl) : 0.f);
    }
  }
  __syncthreads();

  // ---- off-diagonal blocks: one block column per wave, on fp32 matrix cores ----
  // v_mfma_f32_16x16x4f32: lane (l16, g4) supplies A[l16][k] and B[k][l16]
  // for one k of the product's four; D lands as D[4 g4 + i][l16].  Product ks
  // of a 16-wide contraction takes k = 4 g4 + ks, so the result W of the
  // first contraction is, in each lane's registers, exactly the operand
  // W[4 g4 + ks][l16] the second one needs (no trip through LDS), and every
  // A or B fragment of a stored block is the dword 64 ks + lane of its
  // block (the fragment orders above).
  {
    auto column = [&](int dir, int J) {
      const bool up = dir == 1;
      const int I0 = up ? J - 1 : J + 1;
      const int I1 = up ? -1 : NB;
      const int dI = up ? -1 : 1;
      for (int I = I0; I != I1; I += dI) {
        // W = sum_K L_IK T_KJ over K between J and I (T_JJ triangular), in
        // two accumulators (half the dependent chain)
        f32x4 wa[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const int K0 = up ? I + 1 : J, K1 = up ? J : I - 1;
        for (int K = K0; K <= K1; ++K) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int k = 4 * g4 + ks;
            const float av = lblk(I, K)[64 * ks + lane];
            float bv = tblk(K, J)[64 * ks + lane];
            if (K == J && (up ? k > l16 : k < l16)) bv = 0.f;
            wa[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, wa[ks & 1], 0, 0, 0);
          }
        }
        const f32x4 w = wa[0] + wa[1];
        // T_IJ = -T_II W
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          // entry (l16, k) of the diagonal block, read across its B order
          const int k = 4 * g4 + ks;
          float av = tblk(I, I)[64 * (l16 & 3) + 16 * (l16 >> 2) + k];
          if (up ? k < l16 : k > l16) av = 0.f;
          t = __builtin_amdgcn_mfma_f32_16x16x4f32(av, w[ks], t, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) tblk(I, J)[64 * i + lane] = -t[i];
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
    } else if constexpr (NB == 2) {
      if (wave == 0 && fwd_on) column(0, 0);
      if (wave == 1 && rev_on) column(1, 1);
    }  // one block (16-token chunks): no off-diagonal blocks
  }
  __syncthreads();

  // ---- the inverse triangles to the workspace, 16 bytes per store ----
  {
    constexpr int EPS = 16 / (int)sizeof(MT);
    const rsrc_t rt = make_rsrc(static_cast<MT*>(a.tri) + cid * C * C, C * C * (int)sizeof(MT));
    constexpr int NP = C * C / EPS;  // 16-byte pieces of the tile
#pragma unroll
    for (int it = 0; it < (NP + 255) / 256; ++it) {
      const int p = tid + 256 * it;
      if (NP % 256 != 0 && p >= NP) break;
      const int r = (p * EPS) / C, c0 = (p * EPS) % C;
      // EPS consecutive entries of row r, consecutive in its block's B order
      // too.  Every entry is read (all lie inside the tile) and the unused
      // ones are masked away afterwards: a read under the condition would
      // become one branch and one LDS round trip per entry
      const float* src = tblk(r >> 4, c0 >> 4) + 64 * (r & 3) + 16 * ((r >> 2) & 3) + (c0 & 15);
      float tf[EPS];
#pragma unroll
      for (int e = 0; e < EPS; e += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + e);
#pragma unroll
        for (int u = 0; u < 4; ++u) tf[e + u] = v[u];
      }
      MT tv[EPS];
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int col = c0 + e;
        const bool keep = (col < r && fwd_on) || (col > r && rev_on);
        tv[e] = (MT)__uint_as_float(__float_as_uint(tf[e]) & (keep ? ~0u : 0u));
      }
      f32x4 t16;
      __builtin_memcpy(&t16, tv, 16);
      bstore16_ws(ag, rt, p * 16, t16);
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
  // the low parts of the decayed q.k tile exist for bf16 operands only
  const bool plo = std::is_same<MT, bf16>::value && a.pq_lo != nullptr;
  const void* fn = plo ? reinterpret_cast<const void*>(&chunk_prep_kernel<MT, DK, C, true>)
                       : reinterpret_cast<const void*>(&chunk_prep_kernel<MT, DK, C, false>);
  if (query) return hipFuncGetAttributes(query, fn);
  const int64_t G = (a.B * a.H + 7) / 8;
  const int64_t slots = (a.fwd_on && a.rev_on) ? 2 * ((a.NC + 1) / 2) : a.NC;
  // one per chunk id (numbering: see the kernel)
  const int64_t nblocks = a.ready ? slots * G * 8 : (slots * a.B + 7) / 8 * 8 * a.H;
  const dim3 grid((unsigned)nblocks);
  // Beside the state chain, 2 KB more LDS than the kernel declares: a
  // 16-column chain workgroup leaves exactly the kernel's own 37 KB of a
  // compute unit free, and the preparation is kept off the chain's units.
  const unsigned dyn = a.ready ? 2048u : 0u;
  if (plo) hipLaunchKernelGGL((chunk_prep_kernel<MT, DK, C, true>), grid, dim3(256), dyn, stream, a);
  else hipLaunchKernelGGL((chunk_prep_kernel<MT, DK, C, false>), grid, dim3(256), dyn, stream, a);
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
GDN_INST_PREP(float, 64, 16)
GDN_INST_PREP(float, 128, 16)
GDN_INST_PREP(bf16, 64, 16)
GDN_INST_PREP(bf16, 128, 16)

}  // namespace gdn

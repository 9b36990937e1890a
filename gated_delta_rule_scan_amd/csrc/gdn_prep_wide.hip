// Chunk preparation for 128-token chunks: the same state-independent chunk
// quantities as the 32/64-token preparation kernel, in the same workspace
// layout, for a chunk twice as long.
//
// The chunked form is the one every kernel here evaluates ("Video DeltaNet",
// "Key Contributions" item 4: chunk-wise scans with a blocked small-matrix
// inverse kept on chip).  Per chunk and direction, with g the chunk-local
// cumulative log-gate in that direction's visiting order and
// Gamma_ri = exp(g_r - g_i):
//   L    = strictly_lower(diag(beta) (K^K^^T) o Gamma)      (visiting order)
//   Tinv = (I + L)^{-1}
//   P    = (Q^K^^T) o Gamma, the self terms q^_t.k^_t on its diagonal
// In natural token order the forward direction's triangles are lower and the
// reverse direction's upper, so one tile of each holds both directions.
//
// One 512-thread workgroup per (chunk, batch*head) handles both directions.
// At 128 tokens the inverse no longer fits the register and LDS plan of the
// shorter chunks, so this kernel keeps L and the inverse as two fp32 128 x 128
// tiles in LDS (135 KB, one workgroup per compute unit) and takes the plain
// blocked route:
//   1. row norms and raw self terms q.k (four lanes per token), gates; the
//      chunk's raw q and k rows staged in LDS (in the space of the two
//      tiles, before L exists);
//   2. chunk-local cumulative log-gates in double (one wave per direction);
//      the Gram products K K^T and Q K^T on the matrix cores from the staged
//      rows (wave w: row tile w against all eight column tiles);
//   3. L into LDS, the decayed q.k tile to the workspace;
//   4. the sixteen diagonal 16 x 16 blocks of (I + L)^{-1} by substitution,
//      one column per thread; meanwhile the per-token scales;
//   5. the off-diagonal blocks, T_IJ = -T_II sum_K L_IK T_KJ, one block column
//      per direction and wave on fp32 16x16x4 matrix-core products, the
//      column's blocks kept in registers;
//   6. the inverse triangles to the workspace.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kWideC = 128;
constexpr int kWideLP = kWideC + 4;  // fp32 row pitch of the two LDS tiles

// inclusive prefix sum over the 64 lanes of a wave, in double
__device__ __forceinline__ double wave_scan_f64(double x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const double y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Off-diagonal blocks of one block column J of a 128 x 128 unit-triangular
// inverse, on fp32 16x16x4 matrix-core products.  v_mfma_f32_16x16x4f32:
// lane (l16, g4) supplies A[l16][k] and B[k][l16] for one k of the product's
// four; D lands as D[4 g4 + i][l16].  Product ks of a 16-wide contraction
// takes k = 4 g4 + ks, so a result block, as it lands, is in each lane's
// registers exactly the B operand T[4 g4 + ks][l16] of the products that
// read it: the column's blocks stay in registers from one block to the next.
//   forward (lower): T_IJ = -T_II sum_{K=J}^{I-1} L_IK T_KJ, I = J+1 .. 7;
//   reverse (upper): T_IJ = -T_II sum_{K=I+1}^{J} L_IK T_KJ, I = J-1 .. 0.
// Lm holds L and Tm the inverse, both row-major (pitch kWideLP); Tm's
// diagonal blocks are already solved; each result block is stored there too.
template <bool UP, int J>
__device__ __forceinline__ void wide_column(const float* Lm, float* Tm, int lane) {
  constexpr int NB = kWideC / 16, LP = kWideLP;
  const int l16 = lane & 15, g4 = lane >> 4;
  f32x4 tc[NB];  // T_KJ as B operands (K between J and the current block)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int k = 4 * g4 + ks;
    const float d = Tm[(16 * J + k) * LP + 16 * J + l16];  // T_JJ[k][l16]
    tc[J][ks] = (UP ? k <= l16 : k >= l16) ? d : 0.f;    // only its own triangle
  }
  constexpr int NBLK = UP ? J : NB - 1 - J;
#pragma unroll
  for (int n = 0; n < NBLK; ++n) {
    const int I = UP ? J - 1 - n : J + 1 + n;
    const int K0 = UP ? I + 1 : J, K1 = UP ? J : I - 1;
    f32x4 wa[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int K = K0; K <= K1; ++K) {
      const f32x4 lv = *reinterpret_cast<const f32x4*>(&Lm[(16 * I + l16) * LP + 16 * K + 4 * g4]);  // L_IK[l16][4 g4 + ks]
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) wa[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(lv[ks], tc[K][ks], wa[ks & 1], 0, 0, 0);
    }
    const f32x4 w = wa[0] + wa[1];
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    const f32x4 tii = *reinterpret_cast<const f32x4*>(&Tm[(16 * I + l16) * LP + 16 * I + 4 * g4]);  // T_II[l16][4 g4 + ks]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k = 4 * g4 + ks;
      const float av = (UP ? k < l16 : k > l16) ? 0.f : tii[ks];
      t = __builtin_amdgcn_mfma_f32_16x16x4f32(av, w[ks], t, 0, 0, 0);
    }
    tc[I] = -t;
#pragma unroll
    for (int i = 0; i < 4; ++i) Tm[(16 * I + 4 * g4 + i) * LP + 16 * J + l16] = tc[I][i];  // T[16 I + 4 g4 + i][16 J + l16]
  }
}

// Wave w takes the forward column w and the reverse column w + 1 (8 blocks
// between them, whatever w).
template <int W>
__device__ __forceinline__ void wide_columns(const float* Lm, float* Tm, int lane, int fwd_on, int rev_on) {
  if (fwd_on) wide_column<false, W>(Lm, Tm, lane);
  if (rev_on) wide_column<true, W + 1>(Lm, Tm, lane);
}

}  // namespace

// Workgroup barrier for LDS only: this wave's LDS accesses done, then
// s_barrier.  Global loads in flight (the next chunk's rows) stay in flight (a
// __syncthreads() would wait for them); the empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  constexpr int kWaitLds = 0xC07F;  // gfx9 s_waitcnt: lgkmcnt(0), vmcnt and expcnt at their maxima
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitLds);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// A resident grid: workgroup g takes items g, g + gridDim.x, ... (item = one
// (chunk, batch*head)); while it works on one item, the raw q and k rows and
// the gates of its next item are in flight.  Item ids are numbered as
// (chunk, XCD group, XCD): with a grid that is a multiple of eight, a
// sequence's chunks go to the XCD its state-chain workgroups run on.
template <typename MT, int DK>
__global__ __launch_bounds__(512) void chunk_prep_wide_kernel(ScanArgs a, int nitems) {
  using M = Mma<MT>;
  using frag = typename M::frag;
  constexpr int C = kWideC, LP = kWideLP, NB = C / 16;
  constexpr int ES = (int)sizeof(MT);
  constexpr int EP = 16 / ES;       // elements per 16-byte piece
  constexpr int KP = DK + EP;       // row pitch of the staged q and k
  constexpr int EPL = DK / 4;       // elements of a row per lane (four lanes per token)
  constexpr int NPL = EPL * ES / 16;  // 16-byte pieces per lane and matrix
  static_assert((size_t)2 * C * KP * ES <= (size_t)2 * C * LP * 4, "q, k staging fits the two tiles");

  __shared__ __align__(16) float smem[2 * C * LP];
  float* Lm = smem;           // L: forward strictly below, reverse strictly above the diagonal
  float* Tm = smem + C * LP;  // the inverses: forward strictly below, reverse strictly above the diagonal
  // before L exists, the two tiles hold the raw q and k rows of the chunk
  MT* Qs = reinterpret_cast<MT*>(smem);
  MT* Ks = Qs + C * KP;
  __shared__ __align__(16) float s_rk[C], s_rq[C], s_qk[C];
  __shared__ __align__(16) float s_la[2][C], s_bt[2][C];
  __shared__ __align__(16) double s_g[2][C];  // cumulative log2-gates per direction (natural token index)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int nbh = (int)(a.B * a.H), G = (nbh + 7) / 8;
  const int64_t T = a.T, H = a.H, B = a.B;
  const int fwd_on = a.fwd_on, rev_on = a.rev_on;
  const int fslot = 0, rslot = fwd_on ? 1 : 0;
  const size_t nch = (size_t)a.B * a.H * a.NC;
  constexpr double kLog2eD = 1.4426950408889634;
  const float erase_w = a.erase ? 1.f : 0.f;
  const bool ag = ws_agent_stores<C>(a);  // workspace stores at agent scope (see there)
  const uint32_t rowb = (uint32_t)(H * DK * ES);
  const int tok = tid >> 2, part = tid & 3;

  struct Item {
    bool valid;
    int64_t b, h, c, t0, cid;
    int nrows;
  };
  auto item_at = [&](int id) {
    Item it;
    const int64_t bh = (int64_t)((id >> 3) % G) * 8 + (id & 7);
    it.c = (id >> 3) / G;
    it.valid = id < nitems && bh < nbh && it.c < a.NC;
    if (!it.valid) it.c = 0;
    it.b = it.valid ? bh / a.H : 0;
    it.h = it.valid ? bh % a.H : 0;
    it.t0 = it.c * C;
    it.cid = it.valid ? bh * a.NC + it.c : 0;
    it.nrows = it.valid ? (int)(T - it.t0 < C ? T - it.t0 : C) : 1;
    return it;
  };
  // this lane's part of the item's raw q and k rows and its gate (threads
  // 0..255 the log-gates, 256..511 the write strengths, forward then reverse);
  // rows past the sequence, directions that are off and invalid items read zero
  f32x4 vq[NPL], vk[NPL];
  float gv;
  auto fetch = [&](const Item& it) {
    const size_t kq0 = (size_t)((it.b * T + it.t0) * H + it.h) * DK;
    const uint32_t kq_ext = it.valid ? (uint32_t)(it.nrows - 1) * rowb + DK * (uint32_t)ES : 0u;
    const rsrc_t rq = make_rsrc(static_cast<const MT*>(a.q) + kq0, kq_ext);
    const rsrc_t rk = make_rsrc(static_cast<const MT*>(a.k) + kq0, kq_ext);
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const uint32_t off = (uint32_t)tok * rowb + (uint32_t)(part * EPL * ES + 16 * p);
      vq[p] = bload16(rq, off);
      vk[p] = bload16(rk, off);
    }
    const int which = tid / C, t = tid % C;
    const int dir = which & 1;
    const bool on = it.valid && (dir == 0 ? fwd_on : rev_on);
    const int slot = dir == 0 ? fslot : rslot;
    const float* src = which < 2 ? a.log_alpha : a.beta;
    const rsrc_t rg = make_rsrc(src + ((slot * B + it.b) * T + it.t0) * H + it.h,
                                on ? (uint32_t)((it.nrows - 1) * H + 1) * 4u : 0u);
    gv = bload4(rg, (uint32_t)(t * H) * 4u);
  };

  int id = blockIdx.x;
  Item cur = item_at(id);
  fetch(cur);
  for (; id < nitems; id += gridDim.x) {
    const Item nxt = item_at(id + (int)gridDim.x);
    const int64_t b = cur.b, h = cur.h, t0 = cur.t0, cid = cur.cid;
    const int nrows = cur.nrows;

    // ---- 1. row norms, raw self terms and gates; q, k into LDS ----
    {
      float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
      for (int p = 0; p < NPL; ++p) {
        if constexpr (ES == 2) {
          const bf16x8 q8 = __builtin_bit_cast(bf16x8, vq[p]), k8 = __builtin_bit_cast(bf16x8, vk[p]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xq = (float)q8[e], xk = (float)k8[e];
            sq = fmaf(xq, xq, sq);
            sk = fmaf(xk, xk, sk);
            sqk = fmaf(xq, xk, sqk);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sq = fmaf(vq[p][e], vq[p][e], sq);
            sk = fmaf(vk[p][e], vk[p][e], sk);
            sqk = fmaf(vq[p][e], vk[p][e], sqk);
          }
        }
        *reinterpret_cast<f32x4*>(Qs + tok * KP + part * EPL + EP * p) = vq[p];
        *reinterpret_cast<f32x4*>(Ks + tok * KP + part * EPL + EP * p) = vk[p];
      }
#pragma unroll
      for (int m = 1; m < 4; m *= 2) {
        sq += __shfl_xor(sq, m, 64);
        sk += __shfl_xor(sk, m, 64);
        sqk += __shfl_xor(sqk, m, 64);
      }
      if (part == 0) {
        // 1 / max(|x|, eps)
        constexpr float e2 = kNormEps * kNormEps;
        s_rq[tok] = sq > e2 ? 1.0f / sqrtf(sq) : 1.0f / kNormEps;
        s_rk[tok] = sk > e2 ? 1.0f / sqrtf(sk) : 1.0f / kNormEps;
        s_qk[tok] = sqk;
      }
      const int which = tid / C, t = tid % C;
      if (which < 2) s_la[which & 1][t] = gv;
      else s_bt[which & 1][t] = gv;
    }
    // the next item's rows and gates, in flight until its own step 1
    fetch(nxt);
    lds_barrier();

    // ---- 2. cumulative log-gates (waves 0, 1) and the Gram products (all) ----
    // In double: over a fast-decay chunk the sums reach hundreds, where one
    // fp32 rounding is already a relative error of 1e-5 in every decay factor
    // taken as a difference of two of them.  Wave 0: prefix sums in token
    // order; wave 1: suffix sums (the reverse visiting order).  Lane l takes
    // visiting positions 2l and 2l + 1.
    if (wave < 2) {
      const int v0 = 2 * lane, v1 = 2 * lane + 1;
      const int n0 = wave == 0 ? v0 : C - 1 - v0, n1 = wave == 0 ? v1 : C - 1 - v1;  // natural token index
      const double x0 = (double)s_la[wave][n0] * kLog2eD, x1 = (double)s_la[wave][n1] * kLog2eD;
      const double incl = wave_scan_f64(x0 + x1, lane);
      const double excl = incl - (x0 + x1);
      s_g[wave][n0] = excl + x0;
      s_g[wave][n1] = incl;
    }
    // wave w takes row tile ti = w: lane (l16, g4) of tile (ti, tj) ends with
    // row 16 ti + l16 and columns 16 tj + 4 g4 + i (i = 0..3) of K K^T and
    // Q K^T (the products taken transposed), from raw operands
    f32x4 accG[NB], accP[NB];
    {
      const int ti = wave;
      frag qr[DK / 32], kr[DK / 32];
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        qr[ks] = M::load(Qs + (16 * ti + l16) * KP + 32 * ks + 8 * g4);
        kr[ks] = M::load(Ks + (16 * ti + l16) * KP + 32 * ks + 8 * g4);
      }
#pragma unroll
      for (int tj = 0; tj < NB; ++tj) {
        accG[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
        accP[tj] = accG[tj];
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const frag kc = M::load(Ks + (16 * tj + l16) * KP + 32 * ks + 8 * g4);
          accG[tj] = M::mma(kc, kr[ks], accG[tj]);
          accP[tj] = M::mma(kc, qr[ks], accP[tj]);
        }
        // one column tile's reads at a time (hoisted all at once, they would
        // hold 32 fragments in registers)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();  // the q, k staging is reused below

    // ---- 3. L into LDS, the decayed q.k tile to the workspace ----
    {
      const rsrc_t rpq = make_rsrc(static_cast<MT*>(a.pqk) + cid * C * C, cur.valid ? C * C * ES : 0);
      const int r = 16 * wave + l16;
      const float rkr = s_rk[r], rqr = s_rq[r];
      const double gfr = s_g[0][r], grr = s_g[1][r];
      const float flf = rkr * s_bt[0][r] * erase_w, flr = rkr * s_bt[1][r] * erase_w;  // the row's factor of L
      const float self = rqr * rkr * s_qk[r];
#pragma unroll
      for (int tj = 0; tj < NB; ++tj) {
        const int c0 = 16 * tj + 4 * g4;
        // the four columns' k scales and cumulative log-gates, as vectors
        const f32x4 rkc = *reinterpret_cast<const f32x4*>(&s_rk[c0]);
        const double2 gf01 = *reinterpret_cast<const double2*>(&s_g[0][c0]);
        const double2 gf23 = *reinterpret_cast<const double2*>(&s_g[0][c0 + 2]);
        const double2 gr01 = *reinterpret_cast<const double2*>(&s_g[1][c0]);
        const double2 gr23 = *reinterpret_cast<const double2*>(&s_g[1][c0 + 2]);
        const double gfc[4] = {gf01.x, gf01.y, gf23.x, gf23.y}, grc[4] = {gr01.x, gr01.y, gr23.x, gr23.y};
        float pv[4], lv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cc = c0 + i;
          const bool up = cc > r;  // above the diagonal: the reverse direction's entry
          const bool on = up ? rev_on != 0 : (cc < r && fwd_on);
          // decay between the two tokens (<= 0 in log2 units) times the column's k scale
          const float gd = on ? (float)((up ? grr : gfr) - (up ? grc[i] : gfc[i])) : 0.f;
          const float ek = on ? __builtin_amdgcn_exp2f(gd) * rkc[i] : 0.f;
          lv[i] = ((up ? flr : flf) * ek) * accG[tj][i];
          pv[i] = cc == r ? self : (rqr * ek) * accP[tj][i];
        }
        *reinterpret_cast<f32x4*>(&Lm[r * LP + c0]) = f32x4{lv[0], lv[1], lv[2], lv[3]};
        const uint32_t off = (uint32_t)(r * C + c0) * (uint32_t)ES;
        if constexpr (ES == 2) {
          bf16x4 ph;
#pragma unroll
          for (int i = 0; i < 4; ++i) ph[i] = (bf16)pv[i];
          uint32_t w2[2];
          __builtin_memcpy(w2, &ph, 8);
          bstore8_ws(ag, rpq, off, w2[0], w2[1]);
        } else {
          bstore16_ws(ag, rpq, off, f32x4{pv[0], pv[1], pv[2], pv[3]});
        }
      }
    }
    lds_barrier();

    // ---- 4. diagonal blocks of the inverses (threads 0..255), per-token
    // scales and chunk decays (threads 256..511) ----
    if (tid < 2 * NB * 16) {
      const int dir = tid / (NB * 16), blk = (tid / 16) % NB, jc = tid % 16;
      const float* lb = Lm + (16 * blk) * LP + 16 * blk;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = i == jc ? 1.f : 0.f;
      if (dir == 0) {
        if (fwd_on) {
          // column jc of (I + L_bb)^{-1}, L_bb strictly lower: forward substitution
#pragma unroll
          for (int r = 1; r < 16; ++r) {
            float sacc = 0.f;
#pragma unroll
            for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
              const f32x4 lr = *reinterpret_cast<const f32x4*>(lb + r * LP + 4 * i4);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (4 * i4 + e < r) sacc = fmaf(lr[e], x[4 * i4 + e], sacc);
            }
            if (r > jc) x[r] = -sacc;
            // one row's reads at a time (hoisted all at once, they would hold
            // the whole block in registers)
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (i >= jc) Tm[(16 * blk + i) * LP + 16 * blk + jc] = x[i];
        }
      } else if (rev_on) {
        // L_bb strictly upper: backward substitution
#pragma unroll
        for (int r = 14; r >= 0; --r) {
          float sacc = 0.f;
#pragma unroll
          for (int i4 = (r + 1) / 4; i4 < 4; ++i4) {
            const f32x4 lr = *reinterpret_cast<const f32x4*>(lb + r * LP + 4 * i4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * i4 + e > r) sacc = fmaf(lr[e], x[4 * i4 + e], sacc);
          }
          if (r < jc) x[r] = -sacc;
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i <= jc) Tm[(16 * blk + i) * LP + 16 * blk + jc] = x[i];
      }
    } else {
      const int idx = tid - 2 * NB * 16;
      const int dir = idx / C, t = idx % C;
      if (cur.valid && (dir == 0 ? fwd_on : rev_on)) {
        // self term q^_t . k^_t: the operand type's rounding on the diagonal of
        // the decayed q.k tile, the part it drops into each direction's record
        const float rkt = s_rk[t], rqt = s_rq[t];
        const float self = rqt * rkt * s_qk[t];
        const MT self_mt = (MT)self;
        const int slot = dir == 0 ? fslot : rslot;
        const bool in = t < nrows;
        const double g = s_g[dir][t], gl = s_g[dir][dir == 0 ? C - 1 : 0];
        const float eg = exp2f((float)g);
        const rsrc_t rs = make_rsrc(a.sc + (slot * nch + cid) * C, C * 16);
        // {beta, e^g rk (erase term of the pseudo-values; 0 without it), e^g rq, e^(gn-g) rk}
        bstore16_ws(ag, rs, t * 16,
                       in ? f32x4{s_bt[dir][t], a.erase ? eg * rkt : 0.f, eg * rqt, exp2f((float)(gl - g)) * rkt}
                          : f32x4{0.f, 0.f, 0.f, 0.f});
        const rsrc_t rp = make_rsrc(a.pdg + ((size_t)slot * nch + cid) * pdg_stride(C), (C + 4) * 4);
        bstore4_ws(ag, rp, (4 + t) * 4, self - (float)self_mt);
        if (t < 4) bstore4_ws(ag, rp, t * 4, t == 0 ? exp2f((float)gl) : 0.f);
      }
    }
    lds_barrier();

    // ---- 5. off-diagonal blocks on fp32 matrix cores (one block column per
    // direction and wave; see wide_column) ----
    switch (wave) {
      case 0: wide_columns<0>(Lm, Tm, lane, fwd_on, rev_on); break;
      case 1: wide_columns<1>(Lm, Tm, lane, fwd_on, rev_on); break;
      case 2: wide_columns<2>(Lm, Tm, lane, fwd_on, rev_on); break;
      case 3: wide_columns<3>(Lm, Tm, lane, fwd_on, rev_on); break;
      case 4: wide_columns<4>(Lm, Tm, lane, fwd_on, rev_on); break;
      case 5: wide_columns<5>(Lm, Tm, lane, fwd_on, rev_on); break;
      case 6: wide_columns<6>(Lm, Tm, lane, fwd_on, rev_on); break;
      default: break;
    }
    lds_barrier();

    // ---- 6. the inverse triangles to the workspace, 16 bytes per store ----
    {
      constexpr int EPS = 16 / ES;
      constexpr int NP = C * C / EPS;  // 16-byte pieces of the tile
      const rsrc_t rt = make_rsrc(static_cast<MT*>(a.tri) + cid * C * C, cur.valid ? C * C * ES : 0);
#pragma unroll
      for (int it = 0; it < NP / 512; ++it) {
        const int pp = tid + 512 * it;
        const int r = (pp * EPS) / C, c0 = (pp * EPS) % C;
        float x[EPS];
#pragma unroll
        for (int e = 0; e < EPS; e += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&Tm[r * LP + c0 + e]);
#pragma unroll
          for (int u = 0; u < 4; ++u) x[e + u] = v[u];
        }
        MT tv[EPS];
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
          const int col = c0 + e;
          const bool keep = (col < r && fwd_on) || (col > r && rev_on);
          tv[e] = (MT)(keep ? x[e] : 0.f);
        }
        f32x4 t16;
        __builtin_memcpy(&t16, tv, 16);
        bstore16_ws(ag, rt, (uint32_t)(pp * 16), t16);
      }
    }

    // ---- bidirectional scans: the state chain's second visitor recognises
    // an unwritten partial by the all-ones NaN that fills `out` here (a
    // readout never carries it: first visitors store canonical NaNs) ----
    if (a.zero_out && cur.valid) {
      const int sh = 29 - __builtin_clz((unsigned)a.dv);  // log2(dv / 4): 16-byte pieces per row
      const uint32_t orow = (uint32_t)(H * a.dv) * 4u;
      const rsrc_t ro = make_rsrc(a.out + ((b * T + t0) * H + h) * a.dv, (uint32_t)(nrows - 1) * orow + (uint32_t)a.dv * 4u);
      const float fn = __uint_as_float(0xFFFFFFFFu);
      const f32x4 fill = f32x4{fn, fn, fn, fn};
      for (int pp = tid; pp < (C << sh); pp += 512)
        bstore16_ws(ag, ro, (uint32_t)(pp >> sh) * orow + (uint32_t)(pp & ((1 << sh) - 1)) * 16u, fill);
    }

    // ---- publish (concurrent preparation): every store above is
    // agent-scope; once each wave's stores have drained, the chunk's ready
    // flag ----
    if (a.ready) {
      __builtin_amdgcn_s_waitcnt(kWaitVmem);
      __syncthreads();
      if (tid == 0 && cur.valid) __hip_atomic_store(a.ready + cid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    lds_barrier();  // the next item's staging overwrites both tiles
    cur = nxt;
  }
}

template <typename MT, int DK>
hipError_t launch_prep_wide(const ScanArgs& a, hipStream_t stream, hipFuncAttributes* query) {
  const void* fn = reinterpret_cast<const void*>(&chunk_prep_wide_kernel<MT, DK>);
  if (query) return hipFuncGetAttributes(query, fn);
  const int64_t G = (a.B * a.H + 7) / 8;
  const int64_t nitems = a.NC * G * 8;
  // One resident workgroup per compute unit (the two tiles take most of its
  // LDS), a multiple of eight so that an item keeps its XCD.  Beside the
  // state chain (which then holds at most a quarter of the units), half as
  // many, so that every one of them finds a unit at once: a workgroup left
  // waiting for one would hold back the chunks it is dealt.
  const int64_t units = a.ready ? device_compute_units() / 2 : device_compute_units();
  const int64_t ncu = (units + 7) / 8 * 8;
  const dim3 grid((unsigned)(nitems < ncu ? nitems : ncu));
  hipLaunchKernelGGL((chunk_prep_wide_kernel<MT, DK>), grid, dim3(512), 0, stream, a, (int)nitems);
  return hipGetLastError();
}

#define GDN_INST_PREP_WIDE(MT, DK) \
  template hipError_t launch_prep_wide<MT, DK>(const ScanArgs&, hipStream_t, hipFuncAttributes*);
GDN_INST_PREP_WIDE(float, 64)
GDN_INST_PREP_WIDE(float, 128)
GDN_INST_PREP_WIDE(bf16, 64)
GDN_INST_PREP_WIDE(bf16, 128)

}  // namespace gdn

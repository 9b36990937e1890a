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
//   1. row norms and raw self terms q.k (four lanes per token), gates;
//   2. chunk-local cumulative log-gates in double (one wave per direction);
//      the Gram products K K^T and Q K^T on the matrix cores from operands
//      read straight from global memory (eight 16-row tiles per wave);
//   3. L into LDS, the decayed q.k tile to the workspace;
//   4. the sixteen diagonal 16 x 16 blocks of (I + L)^{-1} by substitution,
//      one column per thread; meanwhile the per-token scales;
//   5. the off-diagonal blocks, T_IJ = -T_II sum_K L_IK T_KJ, one block column
//      per direction and wave on fp32 16x16x4 matrix-core products;
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

}  // namespace

template <typename MT, int DK>
__global__ __launch_bounds__(512) void chunk_prep_wide_kernel(ScanArgs a) {
  using M = Mma<MT>;
  using frag = typename M::frag;
  constexpr int C = kWideC, LP = kWideLP, NB = C / 16;
  constexpr int ES = (int)sizeof(MT);

  __shared__ __align__(16) float Lm[C * LP];  // L: forward strictly below, reverse strictly above the diagonal
  __shared__ __align__(16) float Tt[C * LP];  // the inverses, transposed: Tt[c][r] = Tinv[r][c]
  __shared__ __align__(16) float s_rk[C], s_rq[C], s_qk[C];
  __shared__ __align__(16) float s_la[2][C], s_bt[2][C];
  __shared__ __align__(16) double s_g[2][C];  // cumulative log2-gates per direction (natural token index)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  // workgroup id -> (chunk, batch*head): a sequence's chunks go to the XCD
  // its state-chain workgroups run on (ids are dealt round-robin over the
  // eight XCDs)
  const int nbh = (int)(a.B * a.H), G = (nbh + 7) / 8;
  const int id = blockIdx.x;
  const int64_t bh = (int64_t)((id >> 3) % G) * 8 + (id & 7);
  const int64_t c = (id >> 3) / G;
  if (bh >= nbh || c >= a.NC) return;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t T = a.T, H = a.H, B = a.B;
  const int64_t t0 = c * C;
  const int64_t cid = bh * a.NC + c;
  const int fwd_on = a.fwd_on, rev_on = a.rev_on;
  const int fslot = 0, rslot = fwd_on ? 1 : 0;
  const size_t nch = (size_t)a.B * a.H * a.NC;
  const int nrows = (int)(T - t0 < C ? T - t0 : C);  // valid tokens of this chunk (>= 1)
  constexpr double kLog2eD = 1.4426950408889634;
  const float erase_w = a.erase ? 1.f : 0.f;

  // raw q and k of the chunk: rows past the sequence read as zero
  const uint32_t rowb = (uint32_t)(H * DK * ES);
  const size_t kq0 = (size_t)((b * T + t0) * H + h) * DK;
  const uint32_t kq_ext = (uint32_t)(nrows - 1) * rowb + DK * (uint32_t)ES;
  const rsrc_t rq = make_rsrc(static_cast<const MT*>(a.q) + kq0, kq_ext);
  const rsrc_t rk = make_rsrc(static_cast<const MT*>(a.k) + kq0, kq_ext);

  // ---- 1. row norms, raw self terms and gates ----
  {
    const int tok = tid >> 2, part = tid & 3;  // four lanes per token, DK/4 elements each
    constexpr int EPL = DK / 4;
    float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
    for (int p = 0; p < EPL * ES / 16; ++p) {
      const uint32_t off = (uint32_t)tok * rowb + (uint32_t)(part * EPL * ES + 16 * p);
      const f32x4 vq = bload16(rq, off), vk = bload16(rk, off);
      if constexpr (ES == 2) {
        const bf16x8 q8 = __builtin_bit_cast(bf16x8, vq), k8 = __builtin_bit_cast(bf16x8, vk);
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
          sq = fmaf(vq[e], vq[e], sq);
          sk = fmaf(vk[e], vk[e], sk);
          sqk = fmaf(vq[e], vk[e], sqk);
        }
      }
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
    // gates: threads 0..255 the log-gates, 256..511 the write strengths
    // (forward then reverse); tokens past the sequence and directions that
    // are off read zero
    if (tid < 4 * C) {
      const int which = tid / C, t = tid % C;
      const int dir = which & 1;
      const bool on = dir == 0 ? fwd_on : rev_on;
      const int slot = dir == 0 ? fslot : rslot;
      const float* src = which < 2 ? a.log_alpha : a.beta;
      const rsrc_t rg = make_rsrc(src + ((slot * B + b) * T + t0) * H + h, on ? (uint32_t)((nrows - 1) * H + 1) * 4u : 0u);
      const float gv = bload4(rg, (uint32_t)(t * H) * 4u);
      if (which < 2) s_la[dir][t] = gv;
      else s_bt[dir][t] = gv;
    }
  }
  __syncthreads();

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
  // row 16 ti + l16 and columns 16 tj + 4 g4 + i (i = 0..3) of K K^T and Q K^T
  // (the products taken transposed), from raw operands
  f32x4 accG[NB], accP[NB];
  {
    const int ti = wave;
    frag qr[DK / 32], kr[DK / 32];
    const uint32_t orow = (uint32_t)(16 * ti + l16) * rowb + (uint32_t)(8 * g4 * ES);
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      qr[ks] = bload_frag<MT>(rq, orow + 32 * ks * ES);
      kr[ks] = bload_frag<MT>(rk, orow + 32 * ks * ES);
    }
#pragma unroll
    for (int tj = 0; tj < NB; ++tj) {
      accG[tj] = f32x4{0.f, 0.f, 0.f, 0.f};
      accP[tj] = accG[tj];
      const uint32_t ocol = (uint32_t)(16 * tj + l16) * rowb + (uint32_t)(8 * g4 * ES);
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const frag kc = bload_frag<MT>(rk, ocol + 32 * ks * ES);
        accG[tj] = M::mma(kc, kr[ks], accG[tj]);
        accP[tj] = M::mma(kc, qr[ks], accP[tj]);
      }
    }
  }
  __syncthreads();

  // ---- 3. L into LDS, the decayed q.k tile to the workspace ----
  {
    const rsrc_t rpq = make_rsrc(static_cast<MT*>(a.pqk) + cid * C * C, C * C * ES);
    const int r = 16 * wave + l16;
    const float rkr = s_rk[r], rqr = s_rq[r];
    const double gfr = s_g[0][r], grr = s_g[1][r];
    const float flf = rkr * s_bt[0][r] * erase_w, flr = rkr * s_bt[1][r] * erase_w;  // the row's factor of L
    const float self = rqr * rkr * s_qk[r];
#pragma unroll
    for (int tj = 0; tj < NB; ++tj) {
      const int c0 = 16 * tj + 4 * g4;
      float pv[4], lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = c0 + i;
        const bool up = cc > r;  // above the diagonal: the reverse direction's entry
        const bool on = up ? rev_on != 0 : (cc < r && fwd_on);
        // decay between the two tokens (<= 0 in log2 units) times the column's k scale
        const float gd = on ? (float)((up ? grr : gfr) - (up ? s_g[1][cc] : s_g[0][cc])) : 0.f;
        const float ek = on ? __builtin_amdgcn_exp2f(gd) * s_rk[cc] : 0.f;
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
        bstore8_agent(rpq, off, w2[0], w2[1]);
      } else {
        bstore16_agent(rpq, off, f32x4{pv[0], pv[1], pv[2], pv[3]});
      }
    }
  }
  __syncthreads();

  // ---- 4. diagonal blocks of the inverses (threads 0..255), per-token scales
  // and chunk decays (threads 256..511) ----
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
          float s = 0.f;
#pragma unroll
          for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
            const f32x4 lr = *reinterpret_cast<const f32x4*>(lb + r * LP + 4 * i4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * i4 + e < r) s = fmaf(lr[e], x[4 * i4 + e], s);
          }
          if (r > jc) x[r] = -s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i >= jc) Tt[(16 * blk + jc) * LP + 16 * blk + i] = x[i];
      }
    } else if (rev_on) {
      // L_bb strictly upper: backward substitution
#pragma unroll
      for (int r = 14; r >= 0; --r) {
        float s = 0.f;
#pragma unroll
        for (int i4 = (r + 1) / 4; i4 < 4; ++i4) {
          const f32x4 lr = *reinterpret_cast<const f32x4*>(lb + r * LP + 4 * i4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * i4 + e > r) s = fmaf(lr[e], x[4 * i4 + e], s);
        }
        if (r < jc) x[r] = -s;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i <= jc) Tt[(16 * blk + jc) * LP + 16 * blk + i] = x[i];
    }
  } else {
    const int idx = tid - 2 * NB * 16;
    const int dir = idx / C, tok = idx % C;
    if (dir == 0 ? fwd_on : rev_on) {
      // self term q^_t . k^_t: the operand type's rounding on the diagonal of
      // the decayed q.k tile, the part it drops into each direction's record
      const float rkt = s_rk[tok], rqt = s_rq[tok];
      const float self = rqt * rkt * s_qk[tok];
      const MT self_mt = (MT)self;
      const int slot = dir == 0 ? fslot : rslot;
      const bool in = tok < nrows;
      const double g = s_g[dir][tok], gl = s_g[dir][dir == 0 ? C - 1 : 0];
      const float eg = exp2f((float)g);
      const rsrc_t rs = make_rsrc(a.sc + (slot * nch + cid) * C, C * 16);
      // {beta, e^g rk (erase term of the pseudo-values; 0 without it), e^g rq, e^(gn-g) rk}
      bstore16_agent(rs, tok * 16,
                     in ? f32x4{s_bt[dir][tok], a.erase ? eg * rkt : 0.f, eg * rqt, exp2f((float)(gl - g)) * rkt}
                        : f32x4{0.f, 0.f, 0.f, 0.f});
      const rsrc_t rp = make_rsrc(a.pdg + ((size_t)slot * nch + cid) * pdg_stride(C), (C + 4) * 4);
      bstore4_agent(rp, (4 + tok) * 4, self - (float)self_mt);
      if (tok < 4) bstore4_agent(rp, tok * 4, tok == 0 ? exp2f((float)gl) : 0.f);
    }
  }
  __syncthreads();

  // ---- 5. off-diagonal blocks on fp32 matrix cores ----
  // v_mfma_f32_16x16x4f32: lane (l16, g4) supplies A[l16][k] and B[k][l16]
  // for one k of the product's four; D lands as D[4 g4 + i][l16].  Product ks
  // of a 16-wide contraction takes k = 4 g4 + ks, so the result W of the first
  // contraction is, in each lane's registers, the B operand W[4 g4 + ks][l16]
  // of the second one.  Forward (lower): T_IJ = -T_II sum_{K=J}^{I-1} L_IK T_KJ
  // down block column J; reverse (upper): T_IJ = -T_II sum_{K=I+1}^{J} L_IK T_KJ
  // up block column J.  Wave w takes forward column w and reverse column
  // w + 1 (8 blocks each).
  {
    auto column = [&](const bool up, const int J) {
      const int I0 = up ? J - 1 : J + 1, I1 = up ? -1 : NB, dI = up ? -1 : 1;
      for (int I = I0; I != I1; I += dI) {
        f32x4 wa[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const int K0 = up ? I + 1 : J, K1 = up ? J : I - 1;
        for (int K = K0; K <= K1; ++K) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int k = 4 * g4 + ks;
            const float av = Lm[(16 * I + l16) * LP + 16 * K + k];
            float bv = Tt[(16 * J + l16) * LP + 16 * K + k];  // Tinv[16 K + k][16 J + l16]
            // the diagonal block T_JJ: only its own triangle
            if (K == J && (up ? k > l16 : k < l16)) bv = 0.f;
            wa[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, wa[ks & 1], 0, 0, 0);
          }
        }
        const f32x4 w = wa[0] + wa[1];
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int k = 4 * g4 + ks;
          float av = Tt[(16 * I + k) * LP + 16 * I + l16];  // Tinv[16 I + l16][16 I + k]
          if (up ? k < l16 : k > l16) av = 0.f;
          t = __builtin_amdgcn_mfma_f32_16x16x4f32(av, w[ks], t, 0, 0, 0);
        }
        // Tinv[16 I + 4 g4 + i][16 J + l16] = -t[i], stored transposed
        *reinterpret_cast<f32x4*>(&Tt[(16 * J + l16) * LP + 16 * I + 4 * g4]) = f32x4{-t[0], -t[1], -t[2], -t[3]};
      }
    };
    if (wave < NB - 1) {
      if (fwd_on) column(false, wave);
      if (rev_on) column(true, wave + 1);
    }
  }
  __syncthreads();

  // ---- 6. the inverse triangles to the workspace, 16 bytes per store ----
  {
    constexpr int EPS = 16 / ES;
    constexpr int NP = C * C / EPS;  // 16-byte pieces of the tile
    const rsrc_t rt = make_rsrc(static_cast<MT*>(a.tri) + cid * C * C, C * C * ES);
#pragma unroll
    for (int it = 0; it < NP / 512; ++it) {
      const int p = tid + 512 * it;
      const int r = (p * EPS) / C, c0 = (p * EPS) % C;
      MT tv[EPS];
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int col = c0 + e;
        const bool keep = (col < r && fwd_on) || (col > r && rev_on);
        const float x = Tt[col * LP + r];
        tv[e] = (MT)(keep ? x : 0.f);
      }
      f32x4 t16;
      __builtin_memcpy(&t16, tv, 16);
      bstore16_agent(rt, p * 16, t16);
    }
  }

  // ---- bidirectional scans: the state chain's second visitor recognises an
  // unwritten partial by the all-ones NaN that fills `out` here (a readout
  // never carries it: first visitors store canonical NaNs) ----
  if (a.zero_out) {
    const int sh = 29 - __builtin_clz((unsigned)a.dv);  // log2(dv / 4): 16-byte pieces per row
    const uint32_t orow = (uint32_t)(H * a.dv) * 4u;
    const rsrc_t ro = make_rsrc(a.out + ((b * T + t0) * H + h) * a.dv, (uint32_t)(nrows - 1) * orow + (uint32_t)a.dv * 4u);
    const float fn = __uint_as_float(0xFFFFFFFFu);
    const f32x4 fill = f32x4{fn, fn, fn, fn};
    for (int p = tid; p < (C << sh); p += 512)
      bstore16_agent(ro, (uint32_t)(p >> sh) * orow + (uint32_t)(p & ((1 << sh) - 1)) * 16u, fill);
  }

  // ---- publish (concurrent preparation): every store above is agent-scope;
  // once each wave's stores have drained, the chunk's ready flag ----
  if (a.ready) {
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.ready + cid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

template <typename MT, int DK>
hipError_t launch_prep_wide(const ScanArgs& a, hipStream_t stream, hipFuncAttributes* query) {
  const void* fn = reinterpret_cast<const void*>(&chunk_prep_wide_kernel<MT, DK>);
  if (query) return hipFuncGetAttributes(query, fn);
  const int64_t G = (a.B * a.H + 7) / 8;
  const dim3 grid((unsigned)(a.NC * G * 8));
  hipLaunchKernelGGL((chunk_prep_wide_kernel<MT, DK>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

#define GDN_INST_PREP_WIDE(MT, DK) \
  template hipError_t launch_prep_wide<MT, DK>(const ScanArgs&, hipStream_t, hipFuncAttributes*);
GDN_INST_PREP_WIDE(float, 64)
GDN_INST_PREP_WIDE(float, 128)
GDN_INST_PREP_WIDE(bf16, 64)
GDN_INST_PREP_WIDE(bf16, 128)

}  // namespace gdn

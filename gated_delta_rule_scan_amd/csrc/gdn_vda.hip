// Frame-wise delta operator (Video Delta Attention): the memory is written
// once per latent frame as the state closest to the decayed memory that fits
// all of the frame's key-value associations ("Video DeltaNet", "Key
// Contributions" item 2 and "Methodology in Plain English"):
//
//   S_t = (a_t S_{t-1} + B_t) (I + A_t)^{-1},
//   A_t = sum_i beta_i k^_i k^_i^T (dk x dk),  B_t = sum_i beta_i v_i k^_i^T (dv x dk),
//   o_i = S_t q^_i for every token i of frame t.
//
// Three kernels.  Everything that does not depend on the state -- A_t, B_t,
// the inverse M_t = (I + A_t)^{-1} and C_t = B_t M_t -- is computed for all
// frames at once (vda_frame_kernel), so the sequential part is one small
// product per frame, S_t = a_t S_{t-1} M_t + C_t (vda_chain_kernel), and the
// readout runs over all tokens at once (vda_readout_kernel), summing the two
// directions of a bidirectional scan in one store.
//
// M_t is symmetric; the kernels read its rows where a product wants its
// columns (the Gauss-Jordan result is symmetric to rounding).
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

template <typename MT, int DK, int DV>
struct VdaSmem {
  static constexpr bool BF = sizeof(MT) == 2;
  static constexpr int ES = (int)sizeof(MT);
  static constexpr int EP = 16 / ES;           // elements per 16-byte piece
  static constexpr int AP = DK + 4;            // fp32 pitch of the dk x dk and dv x dk matrices
  static constexpr size_t mat_bytes = (size_t)(DK + DV) * AP * 4;
  // one 64-token block: bf16 row-major tiles (read transposed), fp32 transposed tiles
  static constexpr int RP = DK + 8, VP = DV + 8;
  static constexpr int TP = 64 + 4;
  static constexpr size_t stage_bytes = BF ? (size_t)64 * (3 * RP + 2 * VP) * 2 : (size_t)(2 * DK + DV) * TP * 4;
  static constexpr size_t region = mat_bytes > stage_bytes ? mat_bytes : stage_bytes;
};

// ---------------------------------------------------------------------------
// Per frame: A_t and B_t on the matrix cores, M_t by Gauss-Jordan, C_t = B_t M_t.
// One 256-thread workgroup per (direction, batch*head, frame).
// ---------------------------------------------------------------------------
template <typename MT, int DK, int DV>
__global__ __launch_bounds__(256) void vda_frame_kernel(VdaArgs a) {
  using SM = VdaSmem<MT, DK, DV>;
  using M = Mma<MT>;
  using F32 = Mma<float>;
  using frag = typename M::frag;
  constexpr int ES = SM::ES, EP = SM::EP, AP = SM::AP, RP = SM::RP, VP = SM::VP, TP = SM::TP;
  constexpr int NJA = DK / 16 / 4;  // dk tiles of A per wave (row tiles)
  constexpr int NJB = DV / 64;      // dv tiles of B per wave
  constexpr int NL = DK / 16;       // column tiles (dk)
  static_assert(DK % 64 == 0 && DV % 64 == 0, "head dimensions are multiples of 64");

  __shared__ __align__(16) unsigned char smem[SM::region];
  __shared__ float s_wv[64];                   // beta rk of each token of the block
  __shared__ float s_pr[2][DK], s_pc[2][DK];   // Gauss-Jordan pivot row and column

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int NF = (int)a.NF, BH = (int)(a.B * a.H);
  const int f = blockIdx.x % NF;
  const int bh = (blockIdx.x / NF) % BH;
  const int slot = blockIdx.x / (NF * BH);
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t T = a.T, H = a.H, Fr = a.frame;
  const int64_t t0 = (int64_t)f * Fr;
  const int n = (int)(T - t0 < Fr ? T - t0 : Fr);  // tokens of this frame (>= 1)
  const size_t fid = ((size_t)slot * BH + bh) * NF + f;

  f32x4 accA[NJA][NL], accB[NJB][NL];
#pragma unroll
  for (int j = 0; j < NJA; ++j)
#pragma unroll
    for (int l = 0; l < NL; ++l) accA[j][l] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJB; ++j)
#pragma unroll
    for (int l = 0; l < NL; ++l) accB[j][l] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- A_t = K^T diag(beta rk^2) K and B_t = V^T diag(beta rk) K over the
  // frame's tokens, 64 at a time (raw K and V enter the matrix cores; the
  // scaled copies are split hi + lo for bf16 inputs) ----
  constexpr int PRK = DK / EP, RPIK = 256 / PRK, NPK = 64 / RPIK;  // K pieces: per row, rows per pass, per thread
  constexpr int PRV = DV / EP, RPIV = 256 / PRV, NPV = 64 / RPIV;
  const uint32_t HKB = (uint32_t)(H * DK * ES), HVB = (uint32_t)(H * a.dv * ES);
  const int krow = tid / PRK, kcol = (tid % PRK) * EP;
  const int vrow = tid / PRV, vcol = (tid % PRV) * EP;
  MT* Ks = reinterpret_cast<MT*>(smem);        // bf16: [64][RP] raw k, then k w (hi, lo), then v w (hi, lo)
  MT* Kwh = Ks + 64 * RP;
  MT* Kwl = Kwh + 64 * RP;
  MT* Vwh = Kwl + 64 * RP;
  MT* Vwl = Vwh + 64 * VP;
  float* KT = reinterpret_cast<float*>(smem);  // fp32: [DK][TP] raw k^T, then (k w)^T, then (v w)^T
  float* KwT = KT + DK * TP;
  float* VwT = KwT + DK * TP;

  for (int blk = 0; blk < n; blk += 64) {
    const int rows = n - blk < 64 ? n - blk : 64;
    const int64_t tb = t0 + blk;
    const rsrc_t rk = make_rsrc(static_cast<const MT*>(a.k) + ((b * T + tb) * H + h) * DK,
                                (uint32_t)(rows - 1) * HKB + DK * ES);
    const rsrc_t rv = make_rsrc(static_cast<const MT*>(a.v) + ((b * T + tb) * H + h) * a.dv,
                                (uint32_t)(rows - 1) * HVB + (uint32_t)a.dv * ES);
    const rsrc_t rb = make_rsrc(a.beta + ((slot * a.B + b) * T + tb) * H + h, (uint32_t)((rows - 1) * H + 1) * 4u);
    f32x4 kp[NPK], vp[NPV];
    float bk[NPK];
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      kp[i] = bload16(rk, (uint32_t)(krow + RPIK * i) * HKB + kcol * ES);
      bk[i] = bload4(rb, (uint32_t)((krow + RPIK * i) * H) * 4u);
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) vp[i] = bload16(rv, (uint32_t)(vrow + RPIV * i) * HVB + vcol * ES);

    // k rows: norm over the row's lanes, then raw and scaled copies
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      float x[EP], ss = 0.f;
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        if constexpr (SM::BF) {
          x[e] = (float)__builtin_bit_cast(bf16x8, kp[i])[e];
        } else {
          x[e] = kp[i][e];
        }
        ss = fmaf(x[e], x[e], ss);
      }
#pragma unroll
      for (int m = 1; m < PRK; m <<= 1) ss += __shfl_xor(ss, m, 64);
      const float rkn = 1.0f / fmaxf(sqrtf(ss), kNormEps);
      const float wk = bk[i] * rkn * rkn;
      const int row = krow + RPIK * i;
      if (tid % PRK == 0) s_wv[row] = bk[i] * rkn;
      if constexpr (SM::BF) {
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          const float y = wk * x[e];
          hi[e] = (bf16)y;
          lo[e] = (bf16)(y - (float)hi[e]);
        }
        *reinterpret_cast<f32x4*>(Ks + row * RP + kcol) = kp[i];
        *reinterpret_cast<bf16x8*>(Kwh + row * RP + kcol) = hi;
        *reinterpret_cast<bf16x8*>(Kwl + row * RP + kcol) = lo;
      } else {
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          KT[(kcol + e) * TP + row] = x[e];
          KwT[(kcol + e) * TP + row] = wk * x[e];
        }
      }
    }
    __syncthreads();
    // v rows, scaled by beta rk of their token
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int row = vrow + RPIV * i;
      const float wv = s_wv[row];
      if constexpr (SM::BF) {
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          const float y = wv * (float)__builtin_bit_cast(bf16x8, vp[i])[e];
          hi[e] = (bf16)y;
          lo[e] = (bf16)(y - (float)hi[e]);
        }
        *reinterpret_cast<bf16x8*>(Vwh + row * VP + vcol) = hi;
        *reinterpret_cast<bf16x8*>(Vwl + row * VP + vcol) = lo;
      } else {
#pragma unroll
        for (int e = 0; e < EP; ++e) VwT[(vcol + e) * TP + row] = wv * vp[i][e];
      }
    }
    __syncthreads();

    // products: wave w owns dk row tiles NJA w.. of A and dv row tiles NJB w.. of B
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      frag kb[NL];  // raw k^T fragments, one per dk tile
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        if constexpr (SM::BF) {
          kb[l] = load_kt_frag(Ks, RP, 32 * kc, 16 * l, l16, g4);
        } else {
          kb[l] = M::load(KT + (16 * l + l16) * TP + 32 * kc + 8 * g4);
        }
      }
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        if constexpr (SM::BF) {
          const frag wh = load_kt_frag(Kwh, RP, 32 * kc, 16 * l, l16, g4);
          const frag wl = load_kt_frag(Kwl, RP, 32 * kc, 16 * l, l16, g4);
#pragma unroll
          for (int j = 0; j < NJA; ++j) {
            accA[j][l] = M::mma(kb[NJA * w + j], wh, accA[j][l]);
            accA[j][l] = M::mma(kb[NJA * w + j], wl, accA[j][l]);
          }
        } else {
          const frag wk = M::load(KwT + (16 * l + l16) * TP + 32 * kc + 8 * g4);
#pragma unroll
          for (int j = 0; j < NJA; ++j) accA[j][l] = M::mma(kb[NJA * w + j], wk, accA[j][l]);
        }
      }
#pragma unroll
      for (int j = 0; j < NJB; ++j) {
        const int jv = NJB * w + j;
        if constexpr (SM::BF) {
          const frag vh = load_kt_frag(Vwh, VP, 32 * kc, 16 * jv, l16, g4);
          const frag vl = load_kt_frag(Vwl, VP, 32 * kc, 16 * jv, l16, g4);
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            accB[j][l] = M::mma(vh, kb[l], accB[j][l]);
            accB[j][l] = M::mma(vl, kb[l], accB[j][l]);
          }
        } else {
          const frag vw = M::load(VwT + (16 * jv + l16) * TP + 32 * kc + 8 * g4);
#pragma unroll
          for (int l = 0; l < NL; ++l) accB[j][l] = M::mma(vw, kb[l], accB[j][l]);
        }
      }
    }
    __syncthreads();  // the staging area is rewritten by the next block (or the matrices)
  }

  // ---- I + A_t and B_t into LDS (fp32) ----
  float* Am = reinterpret_cast<float*>(smem);  // [DK][AP]
  float* Bm = Am + DK * AP;                    // [DV][AP]
#pragma unroll
  for (int j = 0; j < NJA; ++j)
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * (NJA * w + j) + 4 * g4 + i, c = 16 * l + l16;
        Am[r * AP + c] = accA[j][l][i] + (r == c ? 1.f : 0.f);
      }
#pragma unroll
  for (int j = 0; j < NJB; ++j)
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
      for (int i = 0; i < 4; ++i) Bm[(16 * (NJB * w + j) + 4 * g4 + i) * AP + 16 * l + l16] = accB[j][l][i];
  __syncthreads();

  // ---- M_t = (I + A_t)^{-1}: Gauss-Jordan in place, no pivoting (I + A_t is
  // symmetric positive definite).  Thread (ty, tx) of a 16 x 16 grid keeps a
  // BS x BS block in registers; each pivot's row and column go through LDS
  // (double-buffered: one barrier per pivot). ----
  {
    constexpr int BS = DK / 16;
    const int ty = tid >> 4, tx = tid & 15;
    float m[BS][BS];
#pragma unroll
    for (int i = 0; i < BS; ++i)
#pragma unroll
      for (int j = 0; j < BS; ++j) m[i][j] = Am[(ty * BS + i) * AP + tx * BS + j];
    for (int p = 0; p < DK; ++p) {
      const int buf = p & 1, pb = p / BS, pi = p % BS;
      if (ty == pb) {  // row pi of the block (selects keep the register indices static)
#pragma unroll
        for (int j = 0; j < BS; ++j) {
          float x = 0.f;
#pragma unroll
          for (int ii = 0; ii < BS; ++ii) x = ii == pi ? m[ii][j] : x;
          s_pr[buf][tx * BS + j] = x;
        }
      }
      if (tx == pb) {
#pragma unroll
        for (int i = 0; i < BS; ++i) {
          float x = 0.f;
#pragma unroll
          for (int jj = 0; jj < BS; ++jj) x = jj == pi ? m[i][jj] : x;
          s_pc[buf][ty * BS + i] = x;
        }
      }
      __syncthreads();
      const float d = 1.0f / s_pr[buf][p];
      float r[BS], fc[BS];
#pragma unroll
      for (int j = 0; j < BS; ++j) r[j] = s_pr[buf][tx * BS + j];
#pragma unroll
      for (int i = 0; i < BS; ++i) fc[i] = s_pc[buf][ty * BS + i] * d;
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j) m[i][j] = fmaf(-fc[i], r[j], m[i][j]);
      // the pivot row becomes r d, the pivot column -f d, the pivot d
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j) {
          const bool rowp = ty == pb && i == pi, colp = tx == pb && j == pi;
          m[i][j] = rowp ? (colp ? d : r[j] * d) : (colp ? -fc[i] : m[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < BS; ++i)
#pragma unroll
      for (int j = 0; j < BS; ++j) Am[(ty * BS + i) * AP + tx * BS + j] = m[i][j];
  }
  __syncthreads();

  // ---- C_t^T = M_t B_t^T on fp32 matrix cores (M_t symmetric): tile (l, j)
  // lands in lane (l16, g4) as C_t[16 j + l16][16 l + 4 g4 + i], one 16-byte
  // piece of a row of C_t; M_t rows are written out alongside ----
  {
    float* cg = a.cmat + fid * (size_t)DV * DK;
    constexpr int NLW = NL / 4;  // dk tiles of C^T rows per wave
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
      f32x4 acc[DV / 16];
#pragma unroll
      for (int j = 0; j < DV / 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DK / 32; ++c) {
        const F32::frag mf = F32::load(Am + (16 * l + l16) * AP + 32 * c + 8 * g4);
#pragma unroll
        for (int j = 0; j < DV / 16; ++j)
          acc[j] = F32::mma(mf, F32::load(Bm + (16 * j + l16) * AP + 32 * c + 8 * g4), acc[j]);
      }
#pragma unroll
      for (int j = 0; j < DV / 16; ++j)
        *reinterpret_cast<f32x4*>(cg + (size_t)(16 * j + l16) * DK + 16 * l + 4 * g4) = acc[j];
    }
    float* mg = a.minv + fid * (size_t)DK * DK;
    for (int p = tid; p < DK * DK / 4; p += 256) {
      const int r = p / (DK / 4), c4 = (p % (DK / 4)) * 4;
      *reinterpret_cast<f32x4*>(mg + (size_t)r * DK + c4) = *reinterpret_cast<const f32x4*>(Am + r * AP + c4);
    }
  }
}

// ---------------------------------------------------------------------------
// Sequential over frames: S_t = a_t S_{t-1} M_t + C_t.  One workgroup per
// (direction, batch*head, 16 state rows); the fp32 rows live in LDS.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void vda_chain_kernel(VdaArgs a) {
  using F32 = Mma<float>;
  constexpr int SP = DK + 4;
  constexpr int NLW = DK / 64;  // dk tiles per wave
  __shared__ __align__(16) float Ss[16 * SP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int NF = (int)a.NF, BH = (int)(a.B * a.H), NT = DV / 16;
  const int tile = blockIdx.x % NT;
  const int bh = (blockIdx.x / NT) % BH;
  const int slot = blockIdx.x / (NT * BH);
  const bool rev = a.rev_on && (slot == 1 || !a.fwd_on);
  const int64_t b = bh / a.H, h = bh % a.H;
  const size_t srow = (((size_t)slot * a.B + b) * a.H + h) * DV * DK + (size_t)16 * tile * DK;  // state rows

  for (int p = tid; p < 16 * DK / 4; p += 256) {
    const int r = p / (DK / 4), c4 = (p % (DK / 4)) * 4;
    *reinterpret_cast<f32x4*>(Ss + r * SP + c4) =
        a.state_in ? *reinterpret_cast<const f32x4*>(a.state_in + srow + (size_t)r * DK + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int s = 0; s < NF; ++s) {
    const int f = rev ? NF - 1 - s : s;
    const size_t fid = ((size_t)slot * BH + bh) * NF + f;
    const float* mg = a.minv + fid * (size_t)DK * DK;
    const float* cg = a.cmat + fid * (size_t)DV * DK + (size_t)16 * tile * DK;
    const float at = expf(a.log_alpha[((size_t)slot * a.B + b) * NF * a.H + (size_t)f * a.H + h]);
    __syncthreads();  // Ss holds S_{t-1}
    // (M S^T) tile l lands in lane (l16, g4) as S_new[l16][16 l + 4 g4 + i]
    f32x4 snew[NLW];
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DK / 32; ++c) {
        const F32::frag mf = F32::load(mg + (size_t)(16 * l + l16) * DK + 32 * c + 8 * g4);
        acc = F32::mma(mf, F32::load(Ss + l16 * SP + 32 * c + 8 * g4), acc);
      }
      const f32x4 cv = *reinterpret_cast<const f32x4*>(cg + (size_t)l16 * DK + 16 * l + 4 * g4);
      snew[lw] = acc * at + cv;
    }
    __syncthreads();  // every wave has read S_{t-1}
    float* sg = a.sfr + fid * (size_t)DV * DK + (size_t)16 * tile * DK;
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
      *reinterpret_cast<f32x4*>(Ss + l16 * SP + 16 * l + 4 * g4) = snew[lw];
      *reinterpret_cast<f32x4*>(sg + (size_t)l16 * DK + 16 * l + 4 * g4) = snew[lw];
    }
  }
  __syncthreads();
  if (a.state_out) {
    for (int p = tid; p < 16 * DK / 4; p += 256) {
      const int r = p / (DK / 4), c4 = (p % (DK / 4)) * 4;
      *reinterpret_cast<f32x4*>(a.state_out + srow + (size_t)r * DK + c4) = *reinterpret_cast<const f32x4*>(Ss + r * SP + c4);
    }
  }
}

// ---------------------------------------------------------------------------
// Readout: o_i = S_t q^_i for 64 tokens of one frame per workgroup, both
// directions summed.  Computed transposed (O^T = S_t Q^T, Q raw), so each
// lane holds four consecutive values of one token's output row.
// ---------------------------------------------------------------------------
template <typename MT, int DK, int DV>
__global__ __launch_bounds__(256) void vda_readout_kernel(VdaArgs a, int nblk) {
  using M = Mma<MT>;
  using frag = typename M::frag;
  constexpr int ES = (int)sizeof(MT);
  constexpr int CT = DV / 64;  // dv tiles per wave
  constexpr int KC = DK / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int NF = (int)a.NF, BH = (int)(a.B * a.H);
  const int f = blockIdx.x / nblk, jb = blockIdx.x % nblk;
  const int bh = blockIdx.y;
  const int64_t b = bh / a.H, h = bh % a.H, T = a.T, H = a.H;
  const int64_t fs = (int64_t)f * a.frame + 64 * jb;
  int64_t rows = a.frame - 64 * jb;
  if (T - fs < rows) rows = T - fs;
  if (rows > 64) rows = 64;
  if (rows <= 0) return;
  const uint32_t HQB = (uint32_t)(H * DK * ES), HOB = (uint32_t)(H * DV * 4);
  const rsrc_t rq = make_rsrc(static_cast<const MT*>(a.q) + ((b * T + fs) * H + h) * DK, (uint32_t)(rows - 1) * HQB + DK * ES);
  const rsrc_t ro = make_rsrc(a.out + ((b * T + fs) * H + h) * DV, (uint32_t)(rows - 1) * HOB + DV * 4);

  frag qf[4][KC];
  float rqs[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      qf[rt][c] = bload_frag<MT>(rq, (uint32_t)(16 * rt + l16) * HQB + (32 * c + 8 * g4) * ES);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = M::get(qf[rt][c], e);
        ss = fmaf(x, x, ss);
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    rqs[rt] = 1.0f / fmaxf(sqrtf(ss), kNormEps);
  }
  f32x4 acc[CT][4];
#pragma unroll
  for (int cc = 0; cc < CT; ++cc)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[cc][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int slot = 0; slot < a.dirs; ++slot) {
    const float* sg = a.sfr + (((size_t)slot * BH + bh) * NF + f) * (size_t)DV * DK;
#pragma unroll
    for (int cc = 0; cc < CT; ++cc) {
      const int ct = CT * w + cc;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const float* src = sg + (size_t)(16 * ct + l16) * DK + 32 * c + 8 * g4;
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(src), s1 = *reinterpret_cast<const f32x4*>(src + 4);
        if constexpr (ES == 2) {
          frag hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = e < 4 ? s0[e] : s1[e - 4];
            hi[e] = (bf16)x;
            lo[e] = (bf16)(x - (float)hi[e]);
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            acc[cc][rt] = M::mma(hi, qf[rt][c], acc[cc][rt]);
            acc[cc][rt] = M::mma(lo, qf[rt][c], acc[cc][rt]);
          }
        } else {
          frag sf;
          sf.lo = s0;
          sf.hi = s1;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc[cc][rt] = M::mma(sf, qf[rt][c], acc[cc][rt]);
        }
      }
    }
  }
#pragma unroll
  for (int cc = 0; cc < CT; ++cc)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      bstore16(ro, (uint32_t)(16 * rt + l16) * HOB + (uint32_t)(16 * (CT * w + cc) + 4 * g4) * 4u, acc[cc][rt] * rqs[rt]);
}

template <typename MT, int DK, int DV>
hipError_t launch_vda(const VdaArgs& a, hipStream_t stream, hipEvent_t* ev) {
  const int BH = (int)(a.B * a.H);
  if (a.NF > 0) {
    hipLaunchKernelGGL((vda_frame_kernel<MT, DK, DV>), dim3((unsigned)(a.dirs * BH * a.NF)), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL((vda_chain_kernel<DK, DV>), dim3((unsigned)(a.dirs * BH * (DV / 16))), dim3(256), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return hipErrorLaunchFailure;
  if (a.NF > 0) {
    const int nblk = (int)((a.frame + 63) / 64);
    hipLaunchKernelGGL((vda_readout_kernel<MT, DK, DV>), dim3((unsigned)(a.NF * nblk), (unsigned)BH), dim3(256), 0,
                       stream, a, nblk);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  return hipSuccess;
}

#define GDN_INST_VDA(MT, DK, DV) template hipError_t launch_vda<MT, DK, DV>(const VdaArgs&, hipStream_t, hipEvent_t*);
GDN_INST_VDA(float, 64, 64)
GDN_INST_VDA(float, 64, 128)
GDN_INST_VDA(float, 128, 64)
GDN_INST_VDA(float, 128, 128)
GDN_INST_VDA(bf16, 64, 64)
GDN_INST_VDA(bf16, 64, 128)
GDN_INST_VDA(bf16, 128, 64)
GDN_INST_VDA(bf16, 128, 128)

}  // namespace gdn

// Frame-wise delta operator (Video Delta Attention): the memory is written
// once per latent frame, as the solution of a regularised least-squares
// problem -- the squared distance from the decayed previous memory plus the
// squared recall errors of all the frame's keys ("Video DeltaNet", "Key
// Contributions" item 2 and "Methodology in Plain English"):
//
//   S_t = (a_t S_{t-1} + B_t) (I + A_t)^{-1},
//   A_t = sum_i beta_i k^_i k^_i^T (dk x dk),  B_t = sum_i beta_i v_i k^_i^T (dv x dk),
//   o_i = S_t q^_i for every token i of frame t.
//
// Three kernels.  Everything that does not depend on the state -- A_t, B_t
// and the inverse M_t = (I + A_t)^{-1} -- is computed for all frames at once
// (vda_frame_kernel), so the sequential part is one small product per frame,
// S_t = (a_t S_{t-1} + B_t) M_t (vda_chain_kernel), and the readout runs over
// all tokens at once (vda_readout_kernel), summing the two directions of a
// bidirectional scan in one store.
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
  static constexpr int EP = 16 / ES;            // elements per 16-byte piece
  static constexpr int TB = BF ? 64 : 32;       // tokens per block: one or two matrix-core contractions
  static constexpr int RP = DK + 8, VP = DV + 8;  // bf16 row-major staging pitches
  static constexpr int TP = TB + 4;             // fp32 transposed staging pitch
  static constexpr size_t stage_bytes = BF ? (size_t)TB * (RP + VP) * 2 : (size_t)(DK + DV) * TP * 4;
  static constexpr int AP = DK + 4;             // fp32 pitch of I + A_t
  static constexpr size_t mat_bytes = (size_t)DK * AP * 4;
  // two staging buffers, later reused for I + A_t
  static constexpr size_t region = 2 * stage_bytes > mat_bytes ? 2 * stage_bytes : mat_bytes;
};

// ss + the sum of squares of eight bf16 values (16 bytes), two per
// instruction; bf16 products are exact in fp32
__device__ __forceinline__ float sumsq_bf16x8(const f32x4& p, float ss) {
  // the pairs come from one bit cast of the whole piece and vector shuffles
  // (a bit cast of each extracted float element was compiled to one
  // register for every pair)
  const bf16x8 v = __builtin_bit_cast(bf16x8, p);
  ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), __builtin_shufflevector(v, v, 0, 1), ss, false);
  ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), __builtin_shufflevector(v, v, 2, 3), ss, false);
  ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), __builtin_shufflevector(v, v, 4, 5), ss, false);
  ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), __builtin_shufflevector(v, v, 6, 7), ss, false);
  return ss;
}

// bf16 fragment of raw values times per-token weights (w0: tokens 0-3 of the
// lane's eight, w1: tokens 4-7), split into hi + lo so that the product keeps
// fp32 accuracy on the bf16 matrix cores.
__device__ __forceinline__ void scale_split(const bf16x8& x, const f32x4& w0, const f32x4& w1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = (e < 4 ? w0[e] : w1[e - 4]) * (float)x[e];
    hi[e] = (bf16)y;
    lo[e] = (bf16)(y - (float)hi[e]);
  }
}

// ---------------------------------------------------------------------------
// Per frame: A_t and B_t on the matrix cores, M_t = (I + A_t)^{-1} by
// Gauss-Jordan.  One 256-thread workgroup per (direction, batch*head, frame);
// for two directions the pair of workgroups of one frame is launched
// back-to-back on one XCD, so the second reads the frame's k and v from L2.
// ---------------------------------------------------------------------------
template <typename MT, int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void vda_frame_kernel(VdaArgs a) {
  using SM = VdaSmem<MT, DK, DV>;
  using M = Mma<MT>;
  using frag = typename M::frag;
  constexpr int ES = SM::ES, EP = SM::EP, AP = SM::AP, RP = SM::RP, VP = SM::VP, TP = SM::TP, TB = SM::TB;
  constexpr int NJA = DK / 64;      // dk row tiles of A per wave
  constexpr int NJB = DV / 64;      // dv row tiles of B per wave
  constexpr int NL = DK / 16;       // dk column tiles
  constexpr int TPR = 256 / TB;     // threads per token row when staging
  constexpr int NPK = DK / (TPR * EP), NPV = DV / (TPR * EP);  // 16-byte pieces per thread
  static_assert(DK % 64 == 0 && DV % 64 == 0, "head dimensions are multiples of 64");
  static_assert(NPK >= 1 && NPV >= 1, "staging covers whole rows");

  __shared__ __align__(16) unsigned char smem[SM::region];
  __shared__ __align__(16) float s_wa[2][TB], s_wb[2][TB];  // beta rk^2 (for A) and beta rk (for B) per token
  __shared__ __align__(16) float s_pr[2][DK], s_pc[2][DK];  // Gauss-Jordan pivot row and column

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int NF = (int)a.NF, BH = (int)(a.B * a.H);
  const int64_t U = (int64_t)BH * NF;
  int slot;
  int64_t u;
  if (a.dirs == 2) {
    const int64_t r = blockIdx.x >> 3;
    slot = (int)(r & 1);
    u = (r >> 1) * 8 + (blockIdx.x & 7);
  } else {
    slot = 0;
    u = blockIdx.x;
  }
  if (u >= U) return;  // padding of the last group of eight
  // batch*head fastest: workgroups running together read whole token rows
  // (all heads) of the same frames
  const int bh = (int)(u % BH), f = (int)(u / BH);
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

  // ---- A_t = K^T diag(beta rk^2) K and B_t = V^T diag(beta rk) K, 32 tokens
  // at a time.  Raw k and v are staged (double-buffered, one barrier per
  // block); the weighted side is scaled in registers after the fragment read.
  // Rows past the frame's end read as zero (buffer range checks), weight 0. ----
  const uint32_t HKB = (uint32_t)(H * DK * ES), HVB = (uint32_t)(H * a.dv * ES);
  const int trow = tid / TPR, tpos = tid % TPR;
  f32x4 kp[NPK], vp[NPV];
  float bt;
  auto issue = [&](int blk) {
    const int rows = n - blk < TB ? n - blk : TB;
    const int64_t tb = t0 + blk;
    const rsrc_t rk = make_rsrc(static_cast<const MT*>(a.k) + ((b * T + tb) * H + h) * DK,
                                (uint32_t)(rows - 1) * HKB + DK * ES);
    const rsrc_t rv = make_rsrc(static_cast<const MT*>(a.v) + ((b * T + tb) * H + h) * a.dv,
                                (uint32_t)(rows - 1) * HVB + (uint32_t)a.dv * ES);
    const rsrc_t rb = make_rsrc(a.beta + ((slot * a.B + b) * T + tb) * H + h, (uint32_t)((rows - 1) * H + 1) * 4u);
#pragma unroll
    for (int i = 0; i < NPK; ++i) kp[i] = bload16(rk, (uint32_t)trow * HKB + (uint32_t)((i * TPR + tpos) * EP * ES));
#pragma unroll
    for (int i = 0; i < NPV; ++i) vp[i] = bload16(rv, (uint32_t)trow * HVB + (uint32_t)((i * TPR + tpos) * EP * ES));
    bt = bload4(rb, (uint32_t)(trow * H) * 4u);
  };
  issue(0);
  for (int blk = 0, it = 0; blk < n; blk += TB, ++it) {
    const int buf = it & 1;
    unsigned char* stage = smem + (size_t)buf * SM::stage_bytes;
    // row norm over the row's TPR threads
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      if constexpr (SM::BF) {
        ss = sumsq_bf16x8(kp[i], ss);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(kp[i][e], kp[i][e], ss);
      }
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float rkn = 1.0f / fmaxf(sqrtf(ss), kNormEps);
    if (tpos == 0) {
      s_wa[buf][trow] = bt * rkn * rkn;
      s_wb[buf][trow] = bt * rkn;
    }
    if constexpr (SM::BF) {
      MT* Ks = reinterpret_cast<MT*>(stage);
      MT* Vs = Ks + TB * RP;
#pragma unroll
      for (int i = 0; i < NPK; ++i) *reinterpret_cast<f32x4*>(Ks + trow * RP + (i * TPR + tpos) * EP) = kp[i];
#pragma unroll
      for (int i = 0; i < NPV; ++i) *reinterpret_cast<f32x4*>(Vs + trow * VP + (i * TPR + tpos) * EP) = vp[i];
    } else {
      float* KT = reinterpret_cast<float*>(stage);
      float* VT = KT + DK * TP;
#pragma unroll
      for (int i = 0; i < NPK; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) KT[((i * TPR + tpos) * 4 + e) * TP + trow] = kp[i][e];
#pragma unroll
      for (int i = 0; i < NPV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) VT[((i * TPR + tpos) * 4 + e) * TP + trow] = vp[i][e];
    }
    if (blk + TB < n) issue(blk + TB);
    __syncthreads();

    // the lane's eight tokens of contraction kc are 32 kc + 8 g4 .. + 7 of the block
    if constexpr (SM::BF) {
      const MT* Ks = reinterpret_cast<const MT*>(stage);
      const MT* Vs = Ks + TB * RP;
#pragma unroll
      for (int kc = 0; kc < TB / 32; ++kc) {
        const f32x4 wa0 = *reinterpret_cast<const f32x4*>(&s_wa[buf][32 * kc + 8 * g4]);
        const f32x4 wa1 = *reinterpret_cast<const f32x4*>(&s_wa[buf][32 * kc + 8 * g4 + 4]);
        const f32x4 wb0 = *reinterpret_cast<const f32x4*>(&s_wb[buf][32 * kc + 8 * g4]);
        const f32x4 wb1 = *reinterpret_cast<const f32x4*>(&s_wb[buf][32 * kc + 8 * g4 + 4]);
        frag kr[NL];  // raw k^T, one fragment per dk column tile
#pragma unroll
        for (int l = 0; l < NL; ++l) kr[l] = load_kt_frag(Ks, RP, 32 * kc, 16 * l, l16, g4);
#pragma unroll
        for (int j = 0; j < NJA; ++j) {
          frag xh, xl;
          scale_split(load_kt_frag(Ks, RP, 32 * kc, 16 * (NJA * w + j), l16, g4), wa0, wa1, xh, xl);
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            accA[j][l] = M::mma(xh, kr[l], accA[j][l]);
            accA[j][l] = M::mma(xl, kr[l], accA[j][l]);
          }
        }
#pragma unroll
        for (int j = 0; j < NJB; ++j) {
          frag yh, yl;
          scale_split(load_kt_frag(Vs, VP, 32 * kc, 16 * (NJB * w + j), l16, g4), wb0, wb1, yh, yl);
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            accB[j][l] = M::mma(yh, kr[l], accB[j][l]);
            accB[j][l] = M::mma(yl, kr[l], accB[j][l]);
          }
        }
      }
    } else {
      static_assert(SM::BF || TB == 32, "fp32 staging holds one contraction");
      const f32x4 wa0 = *reinterpret_cast<const f32x4*>(&s_wa[buf][8 * g4]);
      const f32x4 wa1 = *reinterpret_cast<const f32x4*>(&s_wa[buf][8 * g4 + 4]);
      const f32x4 wb0 = *reinterpret_cast<const f32x4*>(&s_wb[buf][8 * g4]);
      const f32x4 wb1 = *reinterpret_cast<const f32x4*>(&s_wb[buf][8 * g4 + 4]);
      const float* KT = reinterpret_cast<const float*>(stage);
      const float* VT = KT + DK * TP;
      frag kr[NL];
#pragma unroll
      for (int l = 0; l < NL; ++l) kr[l] = M::load(KT + (16 * l + l16) * TP + 8 * g4);
#pragma unroll
      for (int j = 0; j < NJA; ++j) {
        frag x = M::load(KT + (16 * (NJA * w + j) + l16) * TP + 8 * g4);
        x.lo *= wa0;
        x.hi *= wa1;
#pragma unroll
        for (int l = 0; l < NL; ++l) accA[j][l] = M::mma(x, kr[l], accA[j][l]);
      }
#pragma unroll
      for (int j = 0; j < NJB; ++j) {
        frag y = M::load(VT + (16 * (NJB * w + j) + l16) * TP + 8 * g4);
        y.lo *= wb0;
        y.hi *= wb1;
#pragma unroll
        for (int l = 0; l < NL; ++l) accB[j][l] = M::mma(y, kr[l], accB[j][l]);
      }
    }
  }
  __syncthreads();  // the staging buffers become I + A_t

  // ---- I + A_t into LDS; B_t straight to the workspace.  Tile (j, l) of a
  // wave holds, in lane (l16, g4), row 16 (tile) + 4 g4 + i, column 16 l + l16.
  // The additive write keeps I - A_t / U (no inverse) and B_t / sqrt(U),
  // U = this frame's token count. ----
  float* Am = reinterpret_cast<float*>(smem);  // [DK][AP]
  const float sa = a.additive ? -1.0f / (float)n : 1.0f;
  const float sb = a.additive ? 1.0f / sqrtf((float)n) : 1.0f;
#pragma unroll
  for (int j = 0; j < NJA; ++j)
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * (NJA * w + j) + 4 * g4 + i, c = 16 * l + l16;
        Am[r * AP + c] = accA[j][l][i] * sa + (r == c ? 1.f : 0.f);
      }
  {
    float* bg = a.bmat + fid * (size_t)DV * DK;
#pragma unroll
    for (int j = 0; j < NJB; ++j)
#pragma unroll
      for (int l = 0; l < NL; ++l)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bg[(size_t)(16 * (NJB * w + j) + 4 * g4 + i) * DK + 16 * l + l16] = accB[j][l][i] * sb;
  }
  __syncthreads();

  // ---- M_t = (I + A_t)^{-1}: Gauss-Jordan in place, no pivoting (I + A_t is
  // symmetric positive definite).  Thread (ty, tx) of a 16 x 16 grid keeps a
  // BS x BS block in registers; each pivot's row and column go through LDS
  // (double-buffered: one barrier per pivot).  The pivot's position inside a
  // block is a compile-time index. ----
  {
    constexpr int BS = DK / 16;
    static_assert(BS % 2 == 0, "pivot buffers alternate within a block");
    const int ty = tid >> 4, tx = tid & 15;
    float m[BS][BS];
#pragma unroll
    for (int i = 0; i < BS; ++i)
#pragma unroll
      for (int j = 0; j < BS; j += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(Am + (ty * BS + i) * AP + tx * BS + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) m[i][j + e] = x[e];
      }
    for (int pb = 0; pb < (a.additive ? 0 : 16); ++pb) {
      const bool rowb = ty == pb, colb = tx == pb;
#pragma unroll
      for (int pi = 0; pi < BS; ++pi) {
        const int buf = pi & 1, p = pb * BS + pi;
        if (rowb) {
#pragma unroll
          for (int j = 0; j < BS; j += 4)
            *reinterpret_cast<f32x4*>(&s_pr[buf][tx * BS + j]) = f32x4{m[pi][j], m[pi][j + 1], m[pi][j + 2], m[pi][j + 3]};
        }
        if (colb) {
#pragma unroll
          for (int i = 0; i < BS; i += 4)
            *reinterpret_cast<f32x4*>(&s_pc[buf][ty * BS + i]) = f32x4{m[i][pi], m[i + 1][pi], m[i + 2][pi], m[i + 3][pi]};
        }
        __syncthreads();
        const float d = 1.0f / s_pr[buf][p];
        float r[BS], fc[BS];
#pragma unroll
        for (int j = 0; j < BS; j += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&s_pr[buf][tx * BS + j]);
          const f32x4 y = *reinterpret_cast<const f32x4*>(&s_pc[buf][ty * BS + j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[j + e] = x[e];
            fc[j + e] = y[e] * d;
          }
        }
#pragma unroll
        for (int i = 0; i < BS; ++i)
#pragma unroll
          for (int j = 0; j < BS; ++j) m[i][j] = fmaf(-fc[i], r[j], m[i][j]);
        // the pivot row becomes r d, the pivot column -f d, the pivot d
#pragma unroll
        for (int j = 0; j < BS; ++j) m[pi][j] = rowb ? r[j] * d : m[pi][j];
#pragma unroll
        for (int i = 0; i < BS; ++i) m[i][pi] = colb ? -fc[i] : m[i][pi];
        m[pi][pi] = rowb && colb ? d : m[pi][pi];
      }
    }
    float* mg = a.minv + fid * (size_t)DK * DK;
    if constexpr (SM::BF) {
      // bf16 inputs: M_t as two bf16 planes, hi then lo (hi + lo = M_t to
      // about 2^-17 relative), the operands of the chain's matrix cores
      bf16* mh = reinterpret_cast<bf16*>(mg);
      bf16* ml = mh + (size_t)DK * DK;
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; j += 4) {
          bf16x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hi[e] = (bf16)m[i][j + e];
            lo[e] = (bf16)(m[i][j + e] - (float)hi[e]);
          }
          const size_t o = (size_t)(ty * BS + i) * DK + tx * BS + j;
          *reinterpret_cast<bf16x4*>(mh + o) = hi;
          *reinterpret_cast<bf16x4*>(ml + o) = lo;
        }
    } else {
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; j += 4)
          *reinterpret_cast<f32x4*>(mg + (size_t)(ty * BS + i) * DK + tx * BS + j) =
              f32x4{m[i][j], m[i][j + 1], m[i][j + 2], m[i][j + 3]};
    }
  }
}

// ---------------------------------------------------------------------------
// Sequential over frames: S_t = R_t M_t with R_t = a_t S_{t-1} + B_t.  One
// workgroup per (direction, batch*head, 16 state rows); R_t's fp32 rows live
// in LDS, and the next frame's M, B and decay are loaded while this frame's
// product runs.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void vda_chain_kernel(VdaArgs a) {
  using F32 = Mma<float>;
  constexpr int SP = DK + 4;
  constexpr int NLW = DK / 64;  // dk tiles per wave
  constexpr int KC = DK / 32;
  __shared__ __align__(16) float Rs[16 * SP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int NF = (int)a.NF, BH = (int)(a.B * a.H), NT = DV / 16;
  // the NT row tiles of one chain share an XCD (workgroup ids equal mod 8), so
  // each frame's M_t is fetched into that XCD's L2 once
  const int g = blockIdx.x >> 3;
  const int tile = g % NT;
  const int chain = (g / NT) * 8 + (blockIdx.x & 7);
  if (chain >= a.dirs * BH) return;
  const int bh = chain % BH;
  const int slot = chain / BH;
  const bool rev = a.rev_on && (slot == 1 || !a.fwd_on);
  const int64_t b = bh / a.H, h = bh % a.H;
  const size_t srow = (((size_t)slot * a.B + b) * a.H + h) * DV * DK + (size_t)16 * tile * DK;  // state rows
  const size_t fbase = ((size_t)slot * BH + bh) * NF;
  const float* lag = a.log_alpha + ((size_t)slot * a.B + b) * NF * a.H + h;

  // the lane's share of a 16 x DK row tile: row l16, columns 16 l + 4 g4 .. + 3.
  // A ring of three register sets holds M, B and the decay of frames s .. s+2:
  // each step consumes one and refills it for frame s + 3 (clamped at the last
  // frame, so every step issues the same loads).
  auto frame_of = [&](int s) { return rev ? NF - 1 - s : s; };
  // B_t enters before the product (R_t = a S + B_t) or, for the additive
  // write, after it (S_t = a S M_t + B_t)
  const float wbefore = a.additive ? 0.f : 1.f, wafter = a.additive ? 1.f : 0.f;
  F32::frag mf[3][NLW][KC];
  f32x4 bn[3][NLW];
  float an[3];
  auto fetch = [&](int k, int s) {
    const int f = frame_of(s < NF ? s : NF - 1);
    const float* mg = a.minv + (fbase + f) * (size_t)DK * DK;
    const float* bg = a.bmat + (fbase + f) * (size_t)DV * DK + (size_t)16 * tile * DK;
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
#pragma unroll
      for (int c = 0; c < KC; ++c) mf[k][lw][c] = F32::load(mg + (size_t)(16 * l + l16) * DK + 32 * c + 8 * g4);
      bn[k][lw] = *reinterpret_cast<const f32x4*>(bg + (size_t)l16 * DK + 16 * l + 4 * g4);
    }
    an[k] = lag[(size_t)f * a.H];
  };
  f32x4 snew[NLW];
#pragma unroll
  for (int lw = 0; lw < NLW; ++lw) {
    const int l = NLW * w + lw;
    snew[lw] = a.state_in ? *reinterpret_cast<const f32x4*>(a.state_in + srow + (size_t)l16 * DK + 16 * l + 4 * g4)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (NF > 0) {
    fetch(0, 0);
    fetch(1, 1);
    fetch(2, 2);
  }
  // drain the prologue's loads: the loop head then sees only the loads of its
  // own previous turn (issued in a fixed order), and waits for no more than it needs
  __builtin_amdgcn_s_waitcnt(kWaitVmem);
  auto step = [&](int s, int k) {
    // keep each step's work inside the step: work hoisted from the next step
    // would wait for loads issued just before
    __builtin_amdgcn_sched_barrier(0);
    const float at = expf(an[k]);
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
      *reinterpret_cast<f32x4*>(Rs + l16 * SP + 16 * l + 4 * g4) = snew[lw] * at + bn[k][lw] * wbefore;
    }
    __syncthreads();  // Rs holds R_t
    // (M R^T) tile l lands in lane (l16, g4) as S_t[l16][16 l + 4 g4 + i]
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) acc = F32::mma(mf[k][lw][c], F32::load(Rs + l16 * SP + 32 * c + 8 * g4), acc);
      snew[lw] = acc + bn[k][lw] * wafter;
    }
    float* sg = a.sfr + (fbase + frame_of(s)) * (size_t)DV * DK + (size_t)16 * tile * DK;
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
      *reinterpret_cast<f32x4*>(sg + (size_t)l16 * DK + 16 * l + 4 * g4) = snew[lw];
    }
    fetch(k, s + 3);
    __syncthreads();  // every wave has read R_t
  };
  // whole turns of the ring, then the remainder (the loop is entered only
  // from full turns, so the wait counts at its head stay exact)
  int s0 = 0;
  for (; s0 + 3 <= NF; s0 += 3) {
    step(s0, 0);
    step(s0 + 1, 1);
    step(s0 + 2, 2);
  }
  if (s0 < NF) step(s0, 0);
  if (s0 + 1 < NF) step(s0 + 1, 1);
  if (a.state_out) {
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
      *reinterpret_cast<f32x4*>(a.state_out + srow + (size_t)l16 * DK + 16 * l + 4 * g4) = snew[lw];
    }
  }
}

// ---------------------------------------------------------------------------
// The same chain for bf16 inputs: 32 state rows per workgroup, and the
// product R_t M_t on the bf16 matrix cores as Rh Mh + Rl Mh + Rh Ml, with
// R_t and M_t split into hi + lo bf16 parts (M_t arrives split from the frame
// kernel; the dropped Rl Ml term is about 2^-16 of the product).  A ring of
// two register sets holds M, B and the decay of frames s and s + 1 (the
// chain streams every frame's M_t and B_t from HBM; a deeper ring does not
// make it faster).
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void vda_chain_bf16_kernel(VdaArgs a) {
  using M = Mma<bf16>;
  using frag = M::frag;
  constexpr int RT = 2;               // 16-row sub-tiles per workgroup
  constexpr int NT = DV / (16 * RT);  // workgroups per chain
  constexpr int NLW = DK / 64;        // output column tiles per wave
  constexpr int KC = DK / 32;         // contraction steps
  constexpr int RP = DK + 8;          // bf16 pitch of R_t's rows
  constexpr int kRing = 2;             // frames in flight
  static_assert(NT >= 1, "dv is a multiple of 32");
  __shared__ __align__(16) bf16 Rh[16 * RT * RP];
  __shared__ __align__(16) bf16 Rl[16 * RT * RP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int NF = (int)a.NF, BH = (int)(a.B * a.H);
  // the NT workgroups of one chain share an XCD (ids equal mod 8)
  const int g = blockIdx.x >> 3;
  const int tile = g % NT;
  const int chain = (g / NT) * 8 + (blockIdx.x & 7);
  if (chain >= a.dirs * BH) return;
  const int bh = chain % BH;
  const int slot = chain / BH;
  const bool rev = a.rev_on && (slot == 1 || !a.fwd_on);
  const int64_t b = bh / a.H, h = bh % a.H;
  const size_t srow = (((size_t)slot * a.B + b) * a.H + h) * DV * DK + (size_t)16 * RT * tile * DK;  // state rows
  const size_t fbase = ((size_t)slot * BH + bh) * NF;
  const float* lag = a.log_alpha + ((size_t)slot * a.B + b) * NF * a.H + h;

  // the lane's share of the 32 x DK row tile: rows 16 rt + l16, columns 16 l + 4 g4 .. + 3
  auto frame_of = [&](int s) { return rev ? NF - 1 - s : s; };
  // B_t enters before the product (R_t = a S + B_t) or, for the additive
  // write, after it (S_t = a S M_t + B_t)
  const float wbefore = a.additive ? 0.f : 1.f, wafter = a.additive ? 1.f : 0.f;
  frag mh[kRing][NLW][KC], ml[kRing][NLW][KC];
  f32x4 bn[kRing][RT][NLW];
  float an[kRing];
  auto fetch = [&](int k, int s) {
    const int f = frame_of(s < NF ? s : NF - 1);
    const bf16* mg = reinterpret_cast<const bf16*>(a.minv + (fbase + f) * (size_t)DK * DK);
    const float* bg = a.bmat + (fbase + f) * (size_t)DV * DK + srow % ((size_t)DV * DK);
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const size_t o = (size_t)(16 * l + l16) * DK + 32 * c + 8 * g4;
        mh[k][lw][c] = M::load(mg + o);
        ml[k][lw][c] = M::load(mg + (size_t)DK * DK + o);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        bn[k][rt][lw] = *reinterpret_cast<const f32x4*>(bg + (size_t)(16 * rt + l16) * DK + 16 * l + 4 * g4);
    }
    an[k] = lag[(size_t)f * a.H];
  };
  f32x4 snew[RT][NLW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int lw = 0; lw < NLW; ++lw) {
      const int l = NLW * w + lw;
      snew[rt][lw] = a.state_in ? *reinterpret_cast<const f32x4*>(a.state_in + srow + (size_t)(16 * rt + l16) * DK +
                                                                    16 * l + 4 * g4)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  if (NF > 0) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) fetch(k, k);
  }
  // drain the prologue's loads: the loop head then sees only the loads of its
  // own previous turn (issued in a fixed order), and waits for no more than it needs
  __builtin_amdgcn_s_waitcnt(kWaitVmem);
  auto step = [&](int s, int k) {
    // keep each step's work inside the step: work hoisted from the next step
    // would wait for loads issued just before
    __builtin_amdgcn_sched_barrier(0);
    const float at = expf(an[k]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int lw = 0; lw < NLW; ++lw) {
        const int l = NLW * w + lw;
        const f32x4 r = snew[rt][lw] * at + bn[k][rt][lw] * wbefore;
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = (bf16)r[e];
          lo[e] = (bf16)(r[e] - (float)hi[e]);
        }
        *reinterpret_cast<bf16x4*>(Rh + (16 * rt + l16) * RP + 16 * l + 4 * g4) = hi;
        *reinterpret_cast<bf16x4*>(Rl + (16 * rt + l16) * RP + 16 * l + 4 * g4) = lo;
      }
    __syncthreads();  // Rh, Rl hold R_t
    // (M R^T) tile (rt, l) lands in lane (l16, g4) as S_t[16 rt + l16][16 l + 4 g4 + i]
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int lw = 0; lw < NLW; ++lw) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const frag rh = M::load(Rh + (16 * rt + l16) * RP + 32 * c + 8 * g4);
          const frag rl = M::load(Rl + (16 * rt + l16) * RP + 32 * c + 8 * g4);
          acc = M::mma(mh[k][lw][c], rh, acc);
          acc = M::mma(mh[k][lw][c], rl, acc);
          acc = M::mma(ml[k][lw][c], rh, acc);
        }
        snew[rt][lw] = acc + bn[k][rt][lw] * wafter;
      }
    // the state store goes out before the next loads, so the wait that frees
    // its registers at the next step does not wait for those loads
    float* sg = a.sfr + (fbase + frame_of(s)) * (size_t)DV * DK + srow % ((size_t)DV * DK);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int lw = 0; lw < NLW; ++lw) {
        const int l = NLW * w + lw;
        *reinterpret_cast<f32x4*>(sg + (size_t)(16 * rt + l16) * DK + 16 * l + 4 * g4) = snew[rt][lw];
      }
    fetch(k, s + kRing);
    __syncthreads();  // every wave has read R_t
  };
  // whole turns of the ring, then the remainder (the loop is entered only
  // from whole turns, so the wait counts at its head stay exact)
  int s0 = 0;
  for (; s0 + kRing <= NF; s0 += kRing) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) step(s0 + k, k);
  }
#pragma unroll
  for (int k = 0; k < kRing - 1; ++k)
    if (s0 + k < NF) step(s0 + k, k);
  if (a.state_out) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int lw = 0; lw < NLW; ++lw) {
        const int l = NLW * w + lw;
        *reinterpret_cast<f32x4*>(a.state_out + srow + (size_t)(16 * rt + l16) * DK + 16 * l + 4 * g4) = snew[rt][lw];
      }
  }
}


// ---------------------------------------------------------------------------
// Readout: o_i = S_t q^_i, both directions summed (o = (S_fwd + S_rev) q^).
// One workgroup per (batch*head, frame, run of 64-token blocks); the summed
// state is split once into the matrix cores' operands and kept in registers
// while the run's blocks stream through LDS.  Computed transposed (O^T = S Q^T,
// Q raw, rows scaled by 1/|q| after), so each lane holds four consecutive
// values of one token's output row; wave w owns the w-th quarter of the dv
// columns.
// ---------------------------------------------------------------------------
template <typename MT, int DK, int DV, bool EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void vda_readout_kernel(VdaArgs a, int nblk,
                                                                                                 int bpw) {
  using M = Mma<MT>;
  using frag = typename M::frag;
  constexpr bool BF = sizeof(MT) == 2;
  constexpr int ES = (int)sizeof(MT);
  constexpr int CT = DV / 64;  // dv tiles per wave
  constexpr int KC = DK / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int NF = (int)a.NF, BH = (int)(a.B * a.H);
  const int nsplit = (nblk + bpw - 1) / bpw;
  // batch*head fastest: workgroups running together cover whole token rows
  const int bh = (int)(blockIdx.x % (unsigned)BH);
  const int fj = (int)(blockIdx.x / (unsigned)BH);
  const int f = fj / nsplit, js = fj % nsplit;
  const int jb0 = js * bpw, jb1 = jb0 + bpw < nblk ? jb0 + bpw : nblk;
  const int64_t b = bh / a.H, h = bh % a.H, T = a.T, H = a.H;
  const int64_t f0 = (int64_t)f * a.frame;
  const int64_t fend = f0 + a.frame < T ? f0 + a.frame : T;
  if (f0 + 64 * (int64_t)jb0 >= fend) return;

  // summed state rows 16 ct + l16, columns 32 c + 8 g4 .. + 7 (every load
  // issued before the first use).  Each direction reads the state after frame
  // f -+ lag (forward: f - lag, reverse: f + lag), or its initial state where
  // that frame does not exist (zero without state_in).
  frag sh[CT][KC];
  [[maybe_unused]] frag sl[CT][KC];
  f32x4 sp[2][CT][KC][2];
  const float* sbase[2];
  float smul[2];
#pragma unroll
  for (int slot = 0; slot < 2; ++slot) {
    const int ss = slot < a.dirs ? slot : 0;
    const bool rev = a.rev_on && (ss == 1 || !a.fwd_on);
    const int src = rev ? f + a.lag : f - a.lag;
    const bool in_range = src >= 0 && src < NF;
    const float* frame_state = a.sfr + (((size_t)ss * BH + bh) * NF + (in_range ? src : 0)) * (size_t)DV * DK;
    sbase[slot] = in_range || !a.state_in ? frame_state : a.state_in + ((size_t)ss * BH + bh) * (size_t)DV * DK;
    // the second direction's part and a missing initial state enter scaled by
    // 0 (a branch here would move the loads behind a wait of their own)
    smul[slot] = (slot < a.dirs && (in_range || a.state_in)) ? 1.f : 0.f;
  }
#pragma unroll
  for (int slot = 0; slot < 2; ++slot)
#pragma unroll
    for (int cc = 0; cc < CT; ++cc)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const float* src = sbase[slot] + (size_t)(16 * (CT * w + cc) + l16) * DK + 32 * c + 8 * g4;
        sp[slot][cc][c][0] = *reinterpret_cast<const f32x4*>(src);
        sp[slot][cc][c][1] = *reinterpret_cast<const f32x4*>(src + 4);
      }
#pragma unroll
  for (int cc = 0; cc < CT; ++cc) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const f32x4 s0 = sp[0][cc][c][0] * smul[0] + sp[1][cc][c][0] * smul[1];
      const f32x4 s1 = sp[0][cc][c][1] * smul[0] + sp[1][cc][c][1] * smul[1];
      if constexpr (BF) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = e < 4 ? s0[e] : s1[e - 4];
          sh[cc][c][e] = (bf16)x;
          sl[cc][c][e] = (bf16)(x - (float)sh[cc][c][e]);
        }
      } else {
        sh[cc][c].lo = s0;
        sh[cc][c].hi = s1;
      }
    }
  }

  const uint32_t HQB = (uint32_t)(H * DK * ES), HOB = (uint32_t)(H * DV * 4), HGB = (uint32_t)(H * DV * ES);
  // epilogue: per-wave sums of squares per token, and this lane's weights
  __shared__ float s_ss[EPI ? 4 : 1][64];
  [[maybe_unused]] f32x4 nw[CT];
  if constexpr (EPI) {
#pragma unroll
    for (int cc = 0; cc < CT; ++cc) nw[cc] = *reinterpret_cast<const f32x4*>(a.norm_weight + 16 * (CT * w + cc) + 4 * g4);
  }
  // blocks jb0 .. jend-1 hold tokens of this frame
  const int64_t nrem = (fend - (f0 + 64 * (int64_t)jb0) + 63) / 64;
  const int jend = jb0 + (int)(nrem < jb1 - jb0 ? nrem : jb1 - jb0);
  auto rows_of = [&](int jb) {
    const int64_t r = fend - (f0 + 64 * (int64_t)jb);
    return (int)(r < 64 ? r : 64);
  };
  // q blocks are staged through LDS (double-buffered): each thread loads its
  // share of a block -- 16-byte pieces, a row's pieces on consecutive threads --
  // kDepth blocks ahead of use, so every wave reads its fragments from LDS
  constexpr int QP = DK + 16 / ES;            // row pitch in elements (16 bytes of padding)
  constexpr int PR = DK * ES / 16;            // 16-byte pieces per row
  constexpr int NPQ = 64 * PR / 256;          // pieces per thread per block
  constexpr int kDepth = BF ? (EPI ? 2 : 3) : 1;  // blocks in flight per thread (the epilogue needs registers)
  __shared__ __align__(16) MT qs[2][64 * QP];
  // bf16 epilogue: the gate logits are staged through LDS beside q, loaded one
  // block ahead (one register set: the q ring holds the rest); fp32 inputs
  // load them per lane at use
  constexpr bool ZST = EPI && BF;
  constexpr int ZP = DV + 16 / ES, PZ = DV * ES / 16, NPZ = ZST ? 64 * PZ / 256 : 1;
  __shared__ __align__(16) MT zs[ZST ? 2 : 1][ZST ? 64 * ZP : 8];
  [[maybe_unused]] f32x4 zr[NPZ];
  auto load_z = [&](int jb, f32x4 (&z)[NPZ]) {
    const int64_t fs = f0 + 64 * (int64_t)jb;
    const rsrc_t rz = make_rsrc(static_cast<const MT*>(a.gate) + ((b * T + fs) * H + h) * DV,
                                (uint32_t)(rows_of(jb) - 1) * HGB + DV * ES);
#pragma unroll
    for (int i = 0; i < NPZ; ++i) {
      const int pc = i * 256 + tid;
      z[i] = bload16(rz, (uint32_t)(pc / PZ) * HGB + (uint32_t)(pc % PZ) * 16u);
    }
  };
  auto load_q = [&](int jb, f32x4 (&qr)[NPQ]) {
    const int64_t fs = f0 + 64 * (int64_t)jb;
    const rsrc_t rq = make_rsrc(static_cast<const MT*>(a.q) + ((b * T + fs) * H + h) * DK,
                                (uint32_t)(rows_of(jb) - 1) * HQB + DK * ES);
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      const int pc = i * 256 + tid;
      qr[i] = bload16(rq, (uint32_t)(pc / PR) * HQB + (uint32_t)(pc % PR) * 16u);
    }
  };
  f32x4 qr[kDepth][NPQ];
  auto block = [&](int jb, int k) {
    __builtin_amdgcn_sched_barrier(0);
    MT* qb = qs[(jb - jb0) & 1];
#pragma unroll
    for (int i = 0; i < NPQ; ++i) {
      const int pc = i * 256 + tid;
      *reinterpret_cast<f32x4*>(qb + (pc / PR) * QP + (pc % PR) * (16 / ES)) = qr[k][i];
    }
    if constexpr (ZST) {
      MT* zb = zs[(jb - jb0) & 1];
#pragma unroll
      for (int i = 0; i < NPZ; ++i) {
        const int pc = i * 256 + tid;
        *reinterpret_cast<f32x4*>(zb + (pc / PZ) * ZP + (pc % PZ) * (16 / ES)) = zr[i];
      }
    }
    // refill this slot kDepth blocks ahead (clamped to the last block); the
    // gate one block ahead
    load_q(jb + kDepth < jend ? jb + kDepth : jend - 1, qr[k]);
    if constexpr (ZST) load_z(jb + 1 < jend ? jb + 1 : jend - 1, zr);
    __syncthreads();  // the block is in LDS; the buffer written two blocks ago is free
    // one 16-token row tile at a time: its fragments, its norms, its products
    f32x4 acc[CT][4];
    float rqs[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      frag qf[KC];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        qf[c] = M::load(qb + (16 * rt + l16) * QP + 32 * c + 8 * g4);
        if constexpr (BF) {
          ss = sumsq_bf16x8(__builtin_bit_cast(f32x4, qf[c]), ss);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(M::get(qf[c], e), M::get(qf[c], e), ss);
        }
      }
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      rqs[rt] = 1.0f / fmaxf(sqrtf(ss), kNormEps);
#pragma unroll
      for (int cc = 0; cc < CT; ++cc) {
        acc[cc][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          acc[cc][rt] = M::mma(sh[cc][c], qf[c], acc[cc][rt]);
          if constexpr (BF) acc[cc][rt] = M::mma(sl[cc][c], qf[c], acc[cc][rt]);
        }
      }
    }
    const int64_t fs = f0 + 64 * (int64_t)jb;
    const rsrc_t ro = make_rsrc(a.out + ((b * T + fs) * H + h) * DV, (uint32_t)(rows_of(jb) - 1) * HOB + DV * 4);
#pragma unroll
    for (int cc = 0; cc < CT; ++cc)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[cc][rt] = acc[cc][rt] * rqs[rt];
    if constexpr (EPI) {
      // epilogue: out = w * o / sqrt(mean(o^2) + eps) * sigmoid(z) per token;
      // the mean over dv spans the four waves (partial sums through LDS)
      [[maybe_unused]] const MT* zb = zs[(jb - jb0) & 1];
      [[maybe_unused]] const rsrc_t rz = make_rsrc(static_cast<const MT*>(a.gate) + ((b * T + fs) * H + h) * DV,
                                                   (uint32_t)(rows_of(jb) - 1) * HGB + DV * ES);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        float ss = 0.f;
#pragma unroll
        for (int cc = 0; cc < CT; ++cc)
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = fmaf(acc[cc][rt][e], acc[cc][rt][e], ss);
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (g4 == 0) s_ss[w][16 * rt + l16] = ss;
      }
      __syncthreads();
      // sigmoid(z) = 1 / (1 + 2^(-z log2 e)) with the hardware exp2 and
      // reciprocal (about 1 ulp each)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float tot = s_ss[0][16 * rt + l16] + s_ss[1][16 * rt + l16] + s_ss[2][16 * rt + l16] + s_ss[3][16 * rt + l16];
        const float inv = 1.0f / sqrtf(tot * (1.0f / DV) + a.norm_eps);
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) {
          // this lane's four gate logits: token 16 rt + l16, columns 16 (CT w + cc) + 4 g4 ..
          f32x4 zv;
          if constexpr (ZST) {
            const uint2 raw = *reinterpret_cast<const uint2*>(zb + (16 * rt + l16) * ZP + 16 * (CT * w + cc) + 4 * g4);
            zv = f32x4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                       __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u)};
          } else {
            zv = bload16(rz, (uint32_t)(16 * rt + l16) * HGB + (uint32_t)(16 * (CT * w + cc) + 4 * g4) * ES);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * zv[e]));
            acc[cc][rt][e] = acc[cc][rt][e] * (inv * nw[cc][e]) * sg;
          }
        }
      }
    }
#pragma unroll
    for (int cc = 0; cc < CT; ++cc)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        bstore16(ro, (uint32_t)(16 * rt + l16) * HOB + (uint32_t)(16 * (CT * w + cc) + 4 * g4) * 4u, acc[cc][rt]);
  };
#pragma unroll
  for (int k = 0; k < kDepth; ++k) {
    load_q(jb0 + k < jend ? jb0 + k : jend - 1, qr[k]);
  }
  if constexpr (ZST) load_z(jb0, zr);
  // whole turns of the ring, then the remainder
  int jb = jb0;
  for (; jb + kDepth <= jend; jb += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) block(jb + k, k);
  }
#pragma unroll
  for (int k = 0; k < kDepth - 1; ++k)
    if (jb + k < jend) block(jb + k, k);
}

template <typename MT, int DK, int DV>
hipError_t launch_vda(const VdaArgs& a, hipStream_t stream, hipEvent_t* ev) {
  const int BH = (int)(a.B * a.H);
  if (a.NF > 0) {
    const int64_t U = (int64_t)BH * a.NF;
    const int64_t grid = a.dirs == 2 ? 2 * ((U + 7) / 8) * 8 : U;
    hipLaunchKernelGGL((vda_frame_kernel<MT, DK, DV>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return hipErrorLaunchFailure;
  {
    const int64_t groups = ((int64_t)a.dirs * BH + 7) / 8;
    if constexpr (sizeof(MT) == 2) {
      hipLaunchKernelGGL((vda_chain_bf16_kernel<DK, DV>), dim3((unsigned)(groups * 8 * (DV / 32))), dim3(256), 0,
                         stream, a);
    } else {
      hipLaunchKernelGGL((vda_chain_kernel<DK, DV>), dim3((unsigned)(groups * 8 * (DV / 16))), dim3(256), 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return hipErrorLaunchFailure;
  if (a.NF > 0) {
    // runs of up to eight 64-token blocks, split evenly over the frame
    const int nblk = (int)((a.frame + 63) / 64);
    const int nsplit = (nblk + 7) / 8;
    const int bpw = (nblk + nsplit - 1) / nsplit;
    const dim3 grid((unsigned)(BH * a.NF * ((nblk + bpw - 1) / bpw)));
    if (a.gate) {
      hipLaunchKernelGGL((vda_readout_kernel<MT, DK, DV, true>), grid, dim3(256), 0, stream, a, nblk, bpw);
    } else {
      hipLaunchKernelGGL((vda_readout_kernel<MT, DK, DV, false>), grid, dim3(256), 0, stream, a, nblk, bpw);
    }
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

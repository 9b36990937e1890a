// Readout epilogue of the token scan ("Video DeltaNet", Key Contributions
// item 1: the linear branch's readout is RMS-normalised and passed through a
// sigmoid gate):
//
//   out[b, t, h, :] = w * o / sqrt(mean_dv(o^2) + eps) * sigmoid(gate[b, t, h, :])
//
// applied in place to the summed readout o that the state chain stored.  The
// mean runs over the dv channels of one (token, head) row; the state chain
// splits those channels over several workgroups (and, bidirectionally, over
// two visits), so the epilogue is its own pass: a streaming kernel that
// reads each row of `out` and `gate` once and writes the row once.
//
// Work split: a row is dv / 2 lanes holding two channels each (dv = 128: a
// whole wave; dv = 64: half a wave), and each lane group keeps kRows rows in
// flight, so the loads of several rows overlap; the sum of squares is a
// butterfly over the row's lanes.  HBM-bound: 10 bytes per channel (fp32 out
// read and written, bf16 gate read; 12 with an fp32 gate).
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kRows = 4;  // rows in flight per lane group

template <typename MT>
__device__ __forceinline__ float2 load_gate2(const MT* p) {
  if constexpr (sizeof(MT) == 2) {
    const uint32_t raw = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(__uint_as_float(raw << 16), __uint_as_float(raw & 0xFFFF0000u));
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

template <typename MT, int DV>
__global__ __launch_bounds__(256) void readout_epilogue_kernel(float* out, const MT* gate, const float* norm_weight,
                                                               float eps, int64_t rows) {
  constexpr int LPR = DV / 2;    // lanes per row
  constexpr int RPW = 64 / LPR;  // rows per wave and pass
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, l = lane % LPR;
  const float2 w = *reinterpret_cast<const float2*>(norm_weight + 2 * l);
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * 256) >> 6;
  for (int64_t r0 = wave * RPW * kRows; r0 < rows; r0 += nwaves * RPW * kRows) {
    float2 o[kRows], z[kRows];
    float ss[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int64_t r = r0 + (int64_t)u * RPW + sub;
      const bool in = r < rows;
      o[u] = in ? *reinterpret_cast<const float2*>(out + r * DV + 2 * l) : make_float2(0.f, 0.f);
      z[u] = in ? load_gate2(gate + r * DV + 2 * l) : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u) ss[u] = fmaf(o[u].x, o[u].x, o[u].y * o[u].y);
    // sum over the row's lanes (butterfly within each group of LPR lanes)
#pragma unroll
    for (int d = LPR / 2; d >= 1; d >>= 1) {
#pragma unroll
      for (int u = 0; u < kRows; ++u) ss[u] += __shfl_xor(ss[u], d, 64);
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int64_t r = r0 + (int64_t)u * RPW + sub;
      if (r < rows) {
        const float inv = 1.0f / sqrtf(ss[u] * (1.0f / DV) + eps);
        float2 y;
        y.x = w.x * (o[u].x * inv) * sigmoid(z[u].x);
        y.y = w.y * (o[u].y * inv) * sigmoid(z[u].y);
        *reinterpret_cast<float2*>(out + r * DV + 2 * l) = y;
      }
    }
  }
}

}  // namespace

template <typename MT, int DV>
hipError_t launch_epilogue(float* out, const void* gate, const float* norm_weight, float eps, int64_t rows,
                           hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  constexpr int RPW = 64 / (DV / 2);
  const int64_t per_block = 4 * RPW * kRows;  // rows a block covers per pass
  int64_t nblocks = (rows + per_block - 1) / per_block;
  if (nblocks > 4096) nblocks = 4096;  // grid-stride beyond: 16 blocks per compute unit
  hipLaunchKernelGGL((readout_epilogue_kernel<MT, DV>), dim3((unsigned)nblocks), dim3(256), 0, stream, out,
                     static_cast<const MT*>(gate), norm_weight, eps, rows);
  return hipGetLastError();
}

template hipError_t launch_epilogue<float, 64>(float*, const void*, const float*, float, int64_t, hipStream_t);
template hipError_t launch_epilogue<float, 128>(float*, const void*, const float*, float, int64_t, hipStream_t);
template hipError_t launch_epilogue<bf16, 64>(float*, const void*, const float*, float, int64_t, hipStream_t);
template hipError_t launch_epilogue<bf16, 128>(float*, const void*, const float*, float, int64_t, hipStream_t);

}  // namespace gdn

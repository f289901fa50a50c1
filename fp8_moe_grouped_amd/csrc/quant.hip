// Activation row quantization of the native FP8 forward ("MoE: native FP8 QAT
// for routed-expert GMMs", Implementation: LHS quantization with one f32 scale
// per row over the full K, max(amax, 1e-12)/448; Description: the activation is
// quantized to e4m3 inside the op).
//
// One wave per row.  The whole bf16 row is held in registers, so it is read
// from HBM once: wave-wide amax -> f32 scale -> correctly rounded f32 quotient
// -> saturating round-to-nearest-even e4m3fn code.  Rows at or past the valid
// prefix (sum of group_sizes) are never read.
#include "common.hpp"
#include "launch.hpp"

namespace fp8gmm {

template <int CPL>  // 16-byte chunks (8 bf16) per lane; covers K <= 512 * CPL
__global__ __launch_bounds__(256) void quant_rows_e4m3_kernel(const uint16_t* __restrict__ lhs,
                                                              const int* __restrict__ group_sizes, int G,
                                                              int M, int K, uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int mv = valid_rows(group_sizes, G, M);
  const int row = blockIdx.x * 4 + wave;
  if (row >= mv) return;
  const int nch = K >> 3;
  const v4i* src = reinterpret_cast<const v4i*>(lhs + (size_t)row * K);
  v4i x[CPL];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nch) {
      x[c] = __builtin_nontemporal_load(src + idx);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = (uint32_t)x[c][e];
        amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_lo(w)));
        amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_hi(w)));
      }
    }
  }
  amax = wave_max(amax);
  const float s = __builtin_fmaxf(amax, kAmaxFloor) / kE4M3Max;   // IEEE f32 division
  v2i* dst = reinterpret_cast<v2i*>(codes + (size_t)row * K);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nch) {
      const uint32_t w0 = x[c][0], w1 = x[c][1], w2 = x[c][2], w3 = x[c][3];
      v2i q;
      q[0] = (int)cvt_e4m3x4(bf16_lo(w0) / s, bf16_hi(w0) / s, bf16_lo(w1) / s, bf16_hi(w1) / s);
      q[1] = (int)cvt_e4m3x4(bf16_lo(w2) / s, bf16_hi(w2) / s, bf16_lo(w3) / s, bf16_hi(w3) / s);
      dst[idx] = q;
    }
  }
  if (lane == 0) scales[row] = s;
}

hipError_t launch_quant_rows_e4m3(const uint16_t* lhs, const int* group_sizes, int G, int M, int K,
                                  uint8_t* codes, float* scales, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int nch = K / 8;
  const int cpl = (nch + 63) / 64;
  dim3 grid((M + 3) / 4), block(256);
#define QLAUNCH(C)                                                                                     \
  hipLaunchKernelGGL(quant_rows_e4m3_kernel<C>, grid, block, 0, stream, lhs, group_sizes, G, M, K, codes, \
                     scales)
  if (cpl <= 1) QLAUNCH(1);
  else if (cpl <= 2) QLAUNCH(2);
  else if (cpl <= 4) QLAUNCH(4);
  else if (cpl <= 8) QLAUNCH(8);
  else if (cpl <= 16) QLAUNCH(16);
  else if (cpl <= 32) QLAUNCH(32);
  else return hipErrorInvalidValue;
#undef QLAUNCH
  return hipGetLastError();
}

}  // namespace fp8gmm

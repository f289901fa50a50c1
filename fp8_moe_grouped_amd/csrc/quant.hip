// Activation row quantization of the native FP8 forward ("MoE: native FP8 QAT
// for routed-expert GMMs", Implementation: LHS quantization with one f32 scale
// per row over the full K, max(amax, 1e-12)/448; Description: the activation is
// quantized to e4m3 inside the op).
//
// One wave per row.  The whole bf16 row is held in registers, so it is read
// from HBM once: wave-wide amax -> f32 scale -> correctly rounded f32 quotient
// -> saturating round-to-nearest-even e4m3fn code.  Rows at or past the valid
// prefix (sum of group_sizes) are never read.
//
// The ops-level variants (same page, Implementation: lhs_quant_block_size 512
// or the full K, and a bf16 scale) use one scale per 512 columns and/or round
// the scale to bf16 before dividing.
#include "common.hpp"
#include "launch.hpp"

namespace fp8gmm {

__device__ __forceinline__ float round_to_bf16(float v) {
  return __builtin_bit_cast(float, pack_bf16x2(v, 0.f) << 16);
}

// CPL: 16-byte chunks (8 bf16) per lane; covers K <= 512 * CPL.
// BLOCK: one scale per 512 columns instead of per row (chunk iteration c of
// the wave covers exactly columns [512c, 512c + 512)); scales are [M, nb].
// SBF16: the f32 scale is rounded once more to bf16 (the bf16-scale option).
// ALL: every row of the static buffer, stale rows included (the buffer-wide
// baseline of the backward; nothing else quantizes stale rows).
template <int CPL, bool BLOCK = false, bool SBF16 = false, bool ALL = false>
__global__ __launch_bounds__(256) void quant_rows_e4m3_kernel(const uint16_t* __restrict__ lhs,
                                                              const int* __restrict__ group_sizes, int G,
                                                              int M, int K, uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int mv = ALL ? M : valid_rows(group_sizes, G, M);
  const int row = blockIdx.x * 4 + wave;
  if (row >= mv) return;
  const int nch = K >> 3;
  // The row's chunks come through a buffer range that ends at the row's end:
  // chunks past it read as zeros (no effect on the amax, never stored), so
  // all CPL loads are issued without a branch (behind a per-chunk branch the
  // compiler waits for each load before issuing the next).
  const BufRsrc rsrc = make_rsrc(lhs + (size_t)row * K, (uint32_t)K * 2u);
  v4i x[CPL];
  float amax[BLOCK ? CPL : 1];
#pragma unroll
  for (int c = 0; c < (BLOCK ? CPL : 1); ++c) amax[c] = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c)
    x[c] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)lane * 16u,
                                                                         (uint32_t)c * 1024u, kCpolStream));
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float& am = amax[BLOCK ? c : 0];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = (uint32_t)x[c][e];
      am = __builtin_fmaxf(am, __builtin_fabsf(bf16_lo(w)));
      am = __builtin_fmaxf(am, __builtin_fabsf(bf16_hi(w)));
    }
  }
  // the quotients widen the codes again instead of keeping the amax pass's
  // widened values alive (8 registers per chunk instead of 4)
#pragma unroll
  for (int c = 0; c < CPL; ++c) asm volatile("" : "+v"(x[c]));
  float sc[BLOCK ? CPL : 1];
#pragma unroll
  for (int c = 0; c < (BLOCK ? CPL : 1); ++c) {
    sc[c] = __builtin_fmaxf(wave_max(amax[c]), kAmaxFloor) / kE4M3Max;   // IEEE f32 division
    if (SBF16) sc[c] = round_to_bf16(sc[c]);
  }
  // The quotient comes from the scale's reciprocal (div_by_scale, checked for
  // f32 scales of this form); a bf16-rounded scale or a non-finite one (an Inf
  // in the row) divides directly.
  float rsc[BLOCK ? CPL : 1];
  bool finite = !SBF16;
#pragma unroll
  for (int c = 0; c < (BLOCK ? CPL : 1); ++c) {
    rsc[c] = 1.0f / sc[c];
    finite = finite && __builtin_isfinite(sc[c]);
  }
  v2i* dst = reinterpret_cast<v2i*>(codes + (size_t)row * K);
  auto quantize = [&](auto fast_c) {
    constexpr bool FAST = decltype(fast_c)::value;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int idx = lane + 64 * c;
      if (idx < nch) {
        const float s = sc[BLOCK ? c : 0], r = rsc[BLOCK ? c : 0];
        auto quo = [&](float v) { return FAST ? div_by_scale(v, s, r) : v / s; };
        const uint32_t w0 = x[c][0], w1 = x[c][1], w2 = x[c][2], w3 = x[c][3];
        v2i q;
        q[0] = (int)cvt_e4m3x4(quo(bf16_lo(w0)), quo(bf16_hi(w0)), quo(bf16_lo(w1)), quo(bf16_hi(w1)));
        q[1] = (int)cvt_e4m3x4(quo(bf16_lo(w2)), quo(bf16_hi(w2)), quo(bf16_lo(w3)), quo(bf16_hi(w3)));
        dst[idx] = q;
      }
    }
  };
  if (finite) quantize(std::true_type{});
  else quantize(std::false_type{});
  if (lane == 0) {
    if (BLOCK) {
      const int nb = (K + 511) >> 9;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        if (c < nb) scales[(size_t)row * nb + c] = sc[c];
    } else {
      scales[row] = sc[0];
    }
  }
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

hipError_t launch_quant_rows_e4m3_variant(const uint16_t* lhs, const int* group_sizes, int G, int M, int K,
                                          bool block512, bool scale_bf16, uint8_t* codes, float* scales,
                                          hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int nch = K / 8;
  const int cpl = (nch + 63) / 64;
  dim3 grid((M + 3) / 4), block(256);
#define QLAUNCH(C, B, S)                                                                                     \
  hipLaunchKernelGGL((quant_rows_e4m3_kernel<C, B, S>), grid, block, 0, stream, lhs, group_sizes, G, M, K,   \
                     codes, scales)
#define QPICK(B, S)                     \
  if (cpl <= 1) QLAUNCH(1, B, S);       \
  else if (cpl <= 2) QLAUNCH(2, B, S);  \
  else if (cpl <= 4) QLAUNCH(4, B, S);  \
  else if (cpl <= 8) QLAUNCH(8, B, S);  \
  else if (cpl <= 16) QLAUNCH(16, B, S); \
  else if (cpl <= 32) QLAUNCH(32, B, S); \
  else return hipErrorInvalidValue;
  if (block512) {
    if (scale_bf16) { QPICK(true, true) } else { QPICK(true, false) }
  } else {
    if (scale_bf16) { QPICK(false, true) } else { QPICK(false, false) }
  }
#undef QPICK
#undef QLAUNCH
  return hipGetLastError();
}

hipError_t launch_quant_rows_e4m3_all(const uint16_t* lhs, int M, int K, uint8_t* codes, float* scales,
                                      hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int cpl = (K / 8 + 63) / 64;
  dim3 grid((M + 3) / 4), block(256);
#define QLAUNCH(C)                                                                                           \
  hipLaunchKernelGGL((quant_rows_e4m3_kernel<C, false, false, true>), grid, block, 0, stream, lhs, nullptr, 0, \
                     M, K, codes, scales)
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

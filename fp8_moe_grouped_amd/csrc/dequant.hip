// Standalone weight dequantization ("MoE: native FP8 QAT for routed-expert
// GMMs", Implementation: dequantize_fp8_codes; the result equals the existing
// dequantize path bit for bit): out[g,k,n] = bf16(f32(dec(codes[g,k,n]) *
// scale[g,n])), the f32 product rounded once to bf16.
//
// HBM-bound (1 byte read + 2 bytes written per element).  Each thread turns
// 16 consecutive codes of one row into 16 bf16 values: one 16-byte load, two
// 16-byte stores, 16 scales from L2.
#include "common.hpp"
#include "launch.hpp"

namespace fp8gmm {
namespace {

__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scale, long long K,
                                                      long long N, long long nchunks,
                                                      uint16_t* __restrict__ out) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long nc_row = N >> 4;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nchunks; i += stride) {
    const long long row = i / nc_row;               // row = g * K + k
    const long long g = row / K;
    const long long n0 = (i - row * nc_row) << 4;
    const v4i c = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(codes) + i);
    const v4f* sp = reinterpret_cast<const v4f*>(scale + g * N + n0);
    v4i o0, o1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f s = sp[q];
      const uint32_t w = (uint32_t)c[q];
      const v2f lo = dec_e4m3x2<false>(w);
      const v2f hi = dec_e4m3x2<true>(w);
      const uint32_t p0 = pack_bf16x2(lo[0] * s[0], lo[1] * s[1]);
      const uint32_t p1 = pack_bf16x2(hi[0] * s[2], hi[1] * s[3]);
      if (q < 2) { o0[2 * q] = (int)p0; o0[2 * q + 1] = (int)p1; }
      else { o1[2 * (q - 2)] = (int)p0; o1[2 * (q - 2) + 1] = (int)p1; }
    }
    v4i* op = reinterpret_cast<v4i*>(out) + 2 * i;
    __builtin_nontemporal_store(o0, op);
    __builtin_nontemporal_store(o1, op + 1);
  }
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const float* scale, int G, long long K, long long N, uint16_t* out,
                          hipStream_t stream) {
  const long long nchunks = (long long)G * K * (N / 16);
  if (nchunks == 0) return hipSuccess;
  long long blocks = (nchunks + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scale, K, N, nchunks, out);
  return hipGetLastError();
}

}  // namespace fp8gmm

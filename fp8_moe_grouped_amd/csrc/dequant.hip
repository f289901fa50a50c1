// Standalone weight dequantization ("MoE: native FP8 QAT for routed-expert
// GMMs", Implementation: dequantize_fp8_codes; the result equals the existing
// dequantize path bit for bit): out[g,k,n] = bf16(f32(dec(codes[g,k,n]) *
// scale[g,n])), the f32 product rounded once to bf16.
//
// HBM-bound (1 byte read + 2 bytes written per element).  A block covers 8
// rows (g, k) of one expert (K is a multiple of 8) and 64 8-code chunks of
// those rows; a thread owns one chunk column, loads its 8 scales once and
// turns 2 rows of 8 codes into bf16 (one 8-byte load and one 16-byte store
// per row, both loads in flight together; 2 rows per thread measured faster
// than 1 or 4 or 8).  A wave's store is 1 KB of
// contiguous output: streaming stores that leave cache lines half written
// (16 codes per lane, two stores 32 bytes apart) run at about half the HBM
// write rate.  No integer division per element: the expert is one scalar
// division per block.
#include "common.hpp"
#include "launch.hpp"

namespace fp8gmm {
namespace {

constexpr int kRowsPerBlock = 8;
constexpr int kRowsPerThread = kRowsPerBlock / 4;   // four waves, each on its own rows
constexpr int kChunksPerBlock = 64;

// ALIGNED: K is a multiple of kRowsPerBlock, so a block's rows belong to one expert.
// Otherwise every row looks up its own expert (rows past the end are skipped).
template <bool ALIGNED>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scale, long long rows, long long K,
                                                      int N, uint16_t* __restrict__ out) {
  const int nc_row = N >> 3;
  const int chunk = blockIdx.y * kChunksPerBlock + (threadIdx.x & 63);
  if (chunk >= nc_row) return;
  const long long rb = (long long)blockIdx.x * kRowsPerBlock;
  const long long row0 = rb + (threadIdx.x >> 6);
  v4f s[2];
  if (ALIGNED) {
    const long long g = rb / K;
    const v4f* sp = reinterpret_cast<const v4f*>(scale + (size_t)g * N + (chunk << 3));
#pragma unroll
    for (int q = 0; q < 2; ++q) s[q] = sp[q];
  }
  v2i c[kRowsPerThread];
#pragma unroll
  for (int r = 0; r < kRowsPerThread; ++r)
    if (ALIGNED || row0 + 4 * r < rows)
      c[r] = __builtin_nontemporal_load(reinterpret_cast<const v2i*>(codes + (row0 + 4 * r) * N) + chunk);
#pragma unroll
  for (int r = 0; r < kRowsPerThread; ++r) {
    const long long row = row0 + 4 * r;
    if (!ALIGNED) {
      if (row >= rows) break;
      const v4f* sp = reinterpret_cast<const v4f*>(scale + (size_t)(row / K) * N + (chunk << 3));
#pragma unroll
      for (int q = 0; q < 2; ++q) s[q] = sp[q];
    }
    v4i o;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t w = (uint32_t)c[r][q];
      const v2f lo = dec_e4m3x2<false>(w);
      const v2f hi = dec_e4m3x2<true>(w);
      o[2 * q] = (int)pack_bf16x2(lo[0] * s[q][0], lo[1] * s[q][1]);
      o[2 * q + 1] = (int)pack_bf16x2(hi[0] * s[q][2], hi[1] * s[q][3]);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<v4i*>(out + row * N) + chunk);
  }
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const float* scale, int G, long long K, long long N, uint16_t* out,
                          hipStream_t stream) {
  const long long rows = (long long)G * K;
  if (rows == 0 || N == 0) return hipSuccess;
  // N is a multiple of 16 and G*K*N < 2^40 (checked by the caller)
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock),
                  (unsigned)((N / 8 + kChunksPerBlock - 1) / kChunksPerBlock));
  if (K % kRowsPerBlock == 0)
    hipLaunchKernelGGL(dequant_kernel<true>, grid, dim3(256), 0, stream, codes, scale, rows, K, (int)N, out);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, grid, dim3(256), 0, stream, codes, scale, rows, K, (int)N, out);
  return hipGetLastError();
}

}  // namespace fp8gmm

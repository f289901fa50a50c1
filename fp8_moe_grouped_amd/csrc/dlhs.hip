// Backward dLHS of the routed-expert GMM from FP8 weight codes ("MoE: native
// FP8 QAT for routed-expert GMMs", Description: the dLHS GMM reads the codes
// and dequantizes each tile on chip, no bf16 weight copy is written to HBM,
// and the result is bit-identical to the dequantize path; Implementation: the
// rhs_contract_dequant path with a double-buffered FP8 stage and per-tile
// dequantization fused into the matmul).
//
// dlhs[r, k] = bf16( sum_n dout[r, n] * w[g, k, n] ),
// w[g, k, n] = bf16( f32(dec(codes[g, k, n]) * scale[g, n]) ).
//
// The scale runs along the contraction axis n, so it cannot move to the
// epilogue: each stage's [BN x 64] code tile is loaded from HBM, dequantized
// once per block (exact e4m3 decode, one f32 multiply, round-to-nearest-even
// bf16 -- the arithmetic of dequantize_fp8_codes) and written to LDS as bf16,
// where four waves read it as bf16 MFMA operands.  The same main loop also
// runs with bf16 weights (FROM_CODES = false), which is the bf16 measurement
// arm; fed with dequantize_fp8_codes' output it must reproduce the FP8-code
// result bit for bit, which proves the on-chip tiles equal the standalone
// dequantization.
//
// Tiling: 256 rows x BN output columns per block (BN = 256 or 128), four
// waves of 128 x BN/2, contraction 64 per stage (two 16x16x32 bf16 MFMA
// steps).  Both LDS tiles are [rows][64 bf16] with a 16-byte-chunk XOR
// swizzle.  The MFMA takes the weight as its first operand so each lane owns
// four consecutive output columns of one row.  Group scheduling and the
// never-read / never-written stale rows are as in the forward.
#include "common.hpp"
#include "launch.hpp"

namespace fp8gmm {
namespace {

constexpr int BM = 256;
constexpr int BKN = 64;                 // contraction (n) per stage, bf16 elements
constexpr int kRowBytes = BKN * 2;      // 128 bytes per LDS tile row
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

template <int BN>
constexpr int stage_bytes() { return (BM + BN) * kRowBytes; }
template <int BN>
constexpr int lds_main() { return 2 * stage_bytes<BN>(); }

__device__ __forceinline__ int t_swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

template <bool FROM_CODES, int NJ>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gmm_dlhs_kernel(const uint16_t* __restrict__ dout, const uint8_t* __restrict__ codes,
                     const float* __restrict__ wscale, const uint16_t* __restrict__ wbf16,
                     const int* __restrict__ group_sizes, int G, int M, int K, int N,
                     uint16_t* __restrict__ dlhs, int* status) {
  constexpr int BN = 32 * NJ;
  constexpr int kStage = stage_bytes<BN>();
  // weight chunks per thread per stage: 16 codes (FROM_CODES) or 8 bf16 per chunk
  constexpr int kWChunksRow = FROM_CODES ? BKN / 16 : BKN / 8;
  constexpr int kWLoads = BN * kWChunksRow / kThreads;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* t_start = reinterpret_cast<int*>(smem + lds_main<BN>());
  int* t_end = t_start + G;
  int* t_pre = t_end + G;

  build_group_table(group_sizes, G, M, BM, GroupTable{t_start, t_end, t_pre}, status);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_tiles = K / BN;
  const int T = t_pre[G];
  const int total = T * n_tiles;
  const int b = blockIdx.x;
  if (b >= total) return;

  const int L = xcd_remap(b, total);
  const int width = kGroupM * n_tiles;
  const int first_m = (L / width) * kGroupM;
  const int gsz = min(T - first_m, kGroupM);
  const int mt = first_m + (L % width) % gsz;
  const int nt = (L % width) / gsz;
  const int g = find_group(t_pre, G, mt);
  const int row0 = t_start[g] + (mt - t_pre[g]) * BM;
  const int rows = min(BM, t_end[g] - row0);

  // ---- activation-gradient (dout) loads: 8 x 16 bytes per thread per stage
  const uint16_t* pa[8];
  int a_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = tid + kThreads * j;
    const int r = i >> 3, c = i & 7;
    const int rr = row0 + min(r, rows - 1);
    pa[j] = dout + (size_t)rr * N + c * 8;
    a_off[j] = t_swz(r, c);
  }
  // ---- weight loads
  const size_t wrow0 = (size_t)g * K + (size_t)nt * BN;
  const uint8_t* pw8[kWLoads];
  const uint16_t* pw16[kWLoads];
  int w_off[kWLoads];
  int wc = 0;
#pragma unroll
  for (int j = 0; j < kWLoads; ++j) {
    const int i = tid + kThreads * j;
    const int kk = i / kWChunksRow, c = i % kWChunksRow;
    wc = c;
    if (FROM_CODES) {
      pw8[j] = codes + (wrow0 + kk) * N + c * 16;
      w_off[j] = t_swz(kk, 2 * c);          // 16 codes -> two 16-byte bf16 chunks
    } else {
      pw16[j] = wbf16 + (wrow0 + kk) * N + c * 8;
      w_off[j] = t_swz(kk, c);
    }
  }
  const float* psc = wscale + (size_t)g * N + wc * 16;   // FROM_CODES: same 16 scales for all chunks

  // ---- MFMA operand read offsets (16x16x32 bf16: lane row l%16, 8 contraction values)
  int a_rd[8][2], b_rd[NJ][2];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int s = 0; s < 2; ++s) a_rd[f][s] = t_swz(wm * 128 + f * 16 + (lane & 15), s * 4 + (lane >> 4));
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int s = 0; s < 2; ++s) b_rd[j][s] = t_swz(wn * (16 * NJ) + j * 16 + (lane & 15), s * 4 + (lane >> 4));

  v4f acc[8][NJ];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  v4i sa[8], sw[kWLoads];
  v4f ssc[4];
  const int nk = N / BKN;

  auto load_stage = [&](int ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sa[j] = *reinterpret_cast<const v4i*>(pa[j] + (size_t)ks * BKN);
    if (FROM_CODES) {
#pragma unroll
      for (int j = 0; j < kWLoads; ++j) sw[j] = *reinterpret_cast<const v4i*>(pw8[j] + (size_t)ks * BKN);
#pragma unroll
      for (int q = 0; q < 4; ++q) ssc[q] = *reinterpret_cast<const v4f*>(psc + (size_t)ks * BKN + 4 * q);
    } else {
#pragma unroll
      for (int j = 0; j < kWLoads; ++j) sw[j] = *reinterpret_cast<const v4i*>(pw16[j] + (size_t)ks * BKN);
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* A = smem + buf * kStage;
    uint8_t* B = A + BM * kRowBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<v4i*>(A + a_off[j]) = sa[j];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
      if (FROM_CODES) {
        // dequantize 16 codes: exact decode, f32 product, RNE to bf16
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = (uint32_t)sw[j][q];
          const v2f lo = dec_e4m3x2<false>(w);
          const v2f hi = dec_e4m3x2<true>(w);
          o[2 * q] = pack_bf16x2(lo[0] * ssc[q][0], lo[1] * ssc[q][1]);
          o[2 * q + 1] = pack_bf16x2(hi[0] * ssc[q][2], hi[1] * ssc[q][3]);
        }
        *reinterpret_cast<v4i*>(B + w_off[j]) = (v4i){(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
        // second 8 values go to the next logical chunk of the same row
        const int kk = (tid + kThreads * j) / kWChunksRow;
        const int c2 = 2 * ((tid + kThreads * j) % kWChunksRow) + 1;
        *reinterpret_cast<v4i*>(B + t_swz(kk, c2)) = (v4i){(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
      } else {
        *reinterpret_cast<v4i*>(B + w_off[j]) = sw[j];
      }
    }
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) load_stage(ks + 1);
    const uint8_t* A = smem + buf * kStage;
    const uint8_t* B = A + BM * kRowBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8bf bfr[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bfr[j] = *reinterpret_cast<const v8bf*>(B + b_rd[j][s]);
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const v8bf af = *reinterpret_cast<const v8bf*>(A + a_rd[f][s]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[f][j] = mfma_bf16_16x16x32(bfr[j], af, acc[f][j]);
      }
    }
    if (ks + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane owns row f*16 + lane%16, columns cb(j) + 4*(lane/16) + 0..3
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int ml = wm * 128 + f * 16 + (lane & 15);
    if (ml < rows) {
      uint16_t* orow = dlhs + (size_t)(row0 + ml) * K + nt * BN + wn * (16 * NJ) + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        v2i pk;
        pk[0] = (int)pack_bf16x2(acc[f][j][0], acc[f][j][1]);
        pk[1] = (int)pack_bf16x2(acc[f][j][2], acc[f][j][3]);
        *reinterpret_cast<v2i*>(orow + j * 16) = pk;
      }
    }
  }
}

template <bool FROM_CODES>
hipError_t launch_dlhs_impl(const uint16_t* dout, const uint8_t* codes, const float* scale, const uint16_t* wbf16,
                            const int* group_sizes, int G, int M, int K, int N, uint16_t* dlhs, int* status,
                            hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const long long max_m_tiles = (M + BM - 1) / BM + G;
  const size_t table = sizeof(int) * (3 * (size_t)G + 1);
  if (K % 256 == 0) {
    hipLaunchKernelGGL((gmm_dlhs_kernel<FROM_CODES, 8>), dim3((unsigned)(max_m_tiles * (K / 256))), dim3(kThreads),
                       lds_main<256>() + table, stream, dout, codes, scale, wbf16, group_sizes, G, M, K, N, dlhs,
                       status);
  } else {
    hipLaunchKernelGGL((gmm_dlhs_kernel<FROM_CODES, 4>), dim3((unsigned)(max_m_tiles * (K / 128))), dim3(kThreads),
                       lds_main<128>() + table, stream, dout, codes, scale, wbf16, group_sizes, G, M, K, N, dlhs,
                       status);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gmm_dlhs_fp8(const uint16_t* dout, const uint8_t* codes, const float* scale, const int* group_sizes,
                               int G, int M, int K, int N, uint16_t* dlhs, int* status, hipStream_t stream) {
  return launch_dlhs_impl<true>(dout, codes, scale, nullptr, group_sizes, G, M, K, N, dlhs, status, stream);
}

hipError_t launch_gmm_bf16_dlhs(const uint16_t* dout, const uint16_t* w, const int* group_sizes, int G, int M, int K,
                                int N, uint16_t* dlhs, int* status, hipStream_t stream) {
  return launch_dlhs_impl<false>(dout, nullptr, nullptr, w, group_sizes, G, M, K, N, dlhs, status, stream);
}

}  // namespace fp8gmm

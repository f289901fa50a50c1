// bf16 grouped forward GEMM: the measurement arm of the FP8/bf16 comparison
// ("MoE: native FP8 QAT for routed-expert GMMs", Tests: GMM kernel
// microbenchmark, the bf16 arm gets a weight dequantized to bf16 beforehand
// and needs no activation quantization).
//
// out[r, n] = bf16( sum_k lhs[r, k] * w[g, k, n] ), f32 accumulation.
//
// Same group schedule, block shape (256 x BN) and wave layout as the FP8
// forward; the contraction advances 64 bf16 per stage on 16x16x32 bf16 MFMA.
// The weight tile keeps its natural [k][n] layout in LDS (rows padded by 32
// bytes so the four rows of one transposing read fall on distinct banks) and
// is read with ds_read_tr16_b64 (4 consecutive k of one column per read).
#include "common.hpp"
#include "launch.hpp"

namespace fp8gmm {
namespace {

constexpr int BM = 256;
constexpr int BKE = 64;                 // contraction elements per stage
constexpr int kARow = BKE * 2;          // 128 bytes per activation row
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

template <int BN>
constexpr int w_stride() { return BN * 2 + 32; }
template <int BN>
constexpr int stage_bytes() { return BM * kARow + BKE * w_stride<BN>(); }
template <int BN>
constexpr int lds_main() { return 2 * stage_bytes<BN>(); }

__device__ __forceinline__ int a_swz(int row, int chunk) { return row * kARow + ((chunk ^ (row & 7)) << 4); }

// Transposing read of four consecutive k (rows) of one bf16 column (gfx950):
// within each 16-lane group lane i receives element j from
// addr[4j + (i>>2)] + 2*(i&3) bytes, addr[L] being lane L's address.
__device__ __forceinline__ v2i lds_read_tr16(const void* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4s, const_cast<void*>(p)));
  return __builtin_bit_cast(v2i, v);
}

template <int NJ>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gmm_bf16_fwd_kernel(const uint16_t* __restrict__ lhs, const uint16_t* __restrict__ w,
                         const int* __restrict__ group_sizes, int G, int M, int K, int N,
                         uint16_t* __restrict__ out, int* status) {
  constexpr int BN = 32 * NJ;
  constexpr int kStage = stage_bytes<BN>();
  constexpr int kWChunksRow = BN / 8;                  // 16-byte chunks per weight row
  constexpr int kWLoads = BKE * kWChunksRow / kThreads;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* t_start = reinterpret_cast<int*>(smem + lds_main<BN>());
  int* t_end = t_start + G;
  int* t_pre = t_end + G;

  build_group_table(group_sizes, G, M, BM, GroupTable{t_start, t_end, t_pre}, status);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_tiles = N / BN;
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

  const uint16_t* pa[8];
  int a_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = tid + kThreads * j;
    const int r = i >> 3, c = i & 7;
    pa[j] = lhs + (size_t)(row0 + min(r, rows - 1)) * K + c * 8;
    a_off[j] = a_swz(r, c);
  }
  const uint16_t* pw[kWLoads];
  int w_off[kWLoads];
  const uint16_t* wg = w + (size_t)g * K * N + (size_t)nt * BN;
#pragma unroll
  for (int j = 0; j < kWLoads; ++j) {
    const int i = tid + kThreads * j;
    const int kk = i / kWChunksRow, c = i % kWChunksRow;
    pw[j] = wg + (size_t)kk * N + c * 8;
    w_off[j] = BM * kARow + kk * w_stride<BN>() + c * 16;
  }
  int a_rd[8][2];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int s = 0; s < 2; ++s) a_rd[f][s] = a_swz(wm * 128 + f * 16 + (lane & 15), s * 4 + (lane >> 4));
  // weight fragment j, sub-step s, half h (k0 = s*32 + (lane/16)*8 + 4h): lane L of the
  // 16-lane group supplies &W[k0 + L/4][cb + 4*(L%4)]
  int w_rd[NJ][2][2];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int cb = wn * (16 * NJ) + j * 16;
    const int Lg = lane & 15;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = s * 32 + (lane >> 4) * 8 + 4 * h + (Lg >> 2);
        const int col = cb + 4 * (Lg & 3);
        w_rd[j][s][h] = BM * kARow + kk * w_stride<BN>() + col * 2;
      }
  }

  v4f acc[8][NJ];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  v4i sa[8], sw[kWLoads];
  const int nk = K / BKE;
  const size_t w_step = (size_t)BKE * N;
  auto load_stage = [&](int ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sa[j] = *reinterpret_cast<const v4i*>(pa[j] + (size_t)ks * BKE);
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) sw[j] = *reinterpret_cast<const v4i*>(pw[j] + (size_t)ks * w_step);
  };
  auto store_stage = [&](int buf) {
    uint8_t* S = smem + buf * kStage;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<v4i*>(S + a_off[j]) = sa[j];
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) *reinterpret_cast<v4i*>(S + w_off[j]) = sw[j];
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) load_stage(ks + 1);
    const uint8_t* S = smem + buf * kStage;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8bf bw[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const v2i lo = lds_read_tr16(S + w_rd[j][s][0]);
        const v2i hi = lds_read_tr16(S + w_rd[j][s][1]);
        bw[j] = __builtin_bit_cast(v8bf, (v4i){lo[0], lo[1], hi[0], hi[1]});
      }
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const v8bf af = *reinterpret_cast<const v8bf*>(S + a_rd[f][s]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[f][j] = mfma_bf16_16x16x32(bw[j], af, acc[f][j]);
      }
    }
    if (ks + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int ml = wm * 128 + f * 16 + (lane & 15);
    if (ml < rows) {
      uint16_t* orow = out + (size_t)(row0 + ml) * N + nt * BN + wn * (16 * NJ) + 4 * (lane >> 4);
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

}  // namespace

hipError_t launch_gmm_bf16_fwd(const uint16_t* lhs, const uint16_t* w, const int* group_sizes, int G, int M, int K,
                               int N, uint16_t* out, int* status, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const long long max_m_tiles = (M + BM - 1) / BM + G;
  const size_t table = sizeof(int) * (3 * (size_t)G + 1);
  if (N % 256 == 0)
    hipLaunchKernelGGL(gmm_bf16_fwd_kernel<8>, dim3((unsigned)(max_m_tiles * (N / 256))), dim3(kThreads),
                       lds_main<256>() + table, stream, lhs, w, group_sizes, G, M, K, N, out, status);
  else
    hipLaunchKernelGGL(gmm_bf16_fwd_kernel<4>, dim3((unsigned)(max_m_tiles * (N / 128))), dim3(kThreads),
                       lds_main<128>() + table, stream, lhs, w, group_sizes, G, M, K, N, out, status);
  return hipGetLastError();
}

}  // namespace fp8gmm

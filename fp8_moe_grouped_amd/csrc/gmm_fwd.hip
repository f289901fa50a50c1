// Native FP8 forward grouped matmul ("MoE: native FP8 QAT for routed-expert
// GMMs", Description and Data flow table: the wi/wo forward GMMs run FP8 x FP8
// with f32 accumulation, reading the e4m3 weight codes and the per-channel f32
// scale directly; Implementation: gmm_silu_fp8 fuses SwiGLU into wi).
//
// out[r, n] = bf16( (sum_k dec(aq[r,k]) * dec(codes[g,k,n])) * ascale[r] * wscale[g,n] )
// for every valid row r of expert g; with SwiGLU the columns are [gate | up]
// and out[r, i] = bf16( silu(y[r, i]) * y[r, I + i] ), I = N/2.
//
// Tiling (gfx950): a block owns a 256-row x BN-column output tile of one
// expert, BN = 256 (or 128 when N is not a multiple of 256; for SwiGLU 128
// gate + the matching 128 up columns); four waves own 128 x BN/2 each, i.e.
// 256 (or 128) f32 accumulators per lane held in AGPRs.  K advances 128 bytes
// per step through two LDS stages:
//  * both tiles are copied HBM/L2 -> LDS by buffer loads with the LDS
//    destination (no VGPR staging), issued at the top of the step for the next
//    stage; per-lane offsets are fixed, one scalar offset advances per step;
//  * the activation tile is row-major, the weight tile keeps the natural
//    [k][n] layout; 16-byte chunks are XOR-swizzled so that the operand reads
//    hit distinct banks (gfx950 LDS serves 256 bytes per cycle);
//  * the weight operand is read with the transposing ds_read_tr8_b64, which
//    hands each lane 8 consecutive k of one column, so the N-contiguous codes
//    need no transpose pass;
//  * activation fragment f+1 is read while the 8 MFMAs of fragment f run, and
//    after a mid-step barrier the next stage's weight fragments are read while
//    the last two fragment groups run; scheduling fences keep this order.
// The MFMA is issued with the weight as its first operand, which makes each
// lane own four consecutive output columns of one row: the epilogue scales,
// optionally applies SwiGLU, and stores 8-byte bf16 groups.
//
// Scheduling: every block rebuilds the expert table from group_sizes (a wave
// scan), maps its id to a (global m-tile, n-tile) pair with an XCD-aware,
// m-grouped order, and exits if it has no tile.  Tiles are aligned to each
// expert's first row; rows past an expert's end are never read (the load row
// is clamped inside the expert) and never written.
#include "common.hpp"
#include "launch.hpp"

namespace fp8gmm {
namespace {

constexpr int BM = 256;
constexpr int BK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

template <int BN>
constexpr int stage_bytes() { return BM * BK + BK * BN; }
template <int BN>
constexpr int lds_main() { return 2 * stage_bytes<BN>(); }   // double buffered

// 16-byte chunk swizzles (bank-conflict free operand reads on 64 banks).
__device__ __forceinline__ int a_key(int row) { return (row >> 1) & 7; }
template <int BN>
__device__ __forceinline__ int b_key(int kk) {
  return BN == 256 ? ((kk & 7) | (((kk >> 5) & 1) << 3)) : (((kk >> 1) & 3) | (((kk >> 5) & 1) << 2));
}
__device__ __forceinline__ int a_swz(int row, int chunk) { return row * BK + ((chunk ^ a_key(row)) << 4); }
template <int BN>
__device__ __forceinline__ int b_swz(int kk, int chunk) { return kk * BN + ((chunk ^ b_key<BN>(kk)) << 4); }

// NJ: 16-column MFMA fragments per wave along N (8 -> BN = 256, 4 -> BN = 128).
template <bool SWIGLU, int NJ>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gmm_fp8_fwd_kernel(const uint8_t* __restrict__ aq, const float* __restrict__ ascale,
                        const uint8_t* __restrict__ codes, const float* __restrict__ wscale,
                        const int* __restrict__ group_sizes, int G, int M, int K, int N,
                        uint16_t* __restrict__ out, int* status) {
  constexpr int BN = 32 * NJ;
  constexpr int kStageBytes = stage_bytes<BN>();
  constexpr int kBChunksRow = BN / 16;                  // 16-byte chunks per weight-tile row
  constexpr int kBLoads = BK * kBChunksRow / kThreads;  // weight chunks per thread per stage
  constexpr int kBRowsPerLoad = 1024 / BN;              // weight rows per wave-wide load
  static_assert(!SWIGLU || NJ == 8, "SwiGLU pairs 4 gate with 4 up fragments");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* t_start = reinterpret_cast<int*>(smem + lds_main<BN>());
  int* t_end = t_start + G;
  int* t_pre = t_end + G;

  build_group_table(group_sizes, G, M, BM, GroupTable{t_start, t_end, t_pre}, status);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int I = N >> 1;
  const int n_tiles = SWIGLU ? (I / (BN / 2)) : (N / BN);
  const int T = t_pre[G];
  const int total = T * n_tiles;
  const int b = blockIdx.x;
  if (b >= total) return;

  // ---- tile selection: XCD-aware, groups of kGroupM m-tiles walk the n-tiles
  const int L = xcd_remap(b, total);
  const int width = kGroupM * n_tiles;
  const int first_m = (L / width) * kGroupM;
  const int gsz = min(T - first_m, kGroupM);
  const int mt = first_m + (L % width) % gsz;
  // values read from the LDS table are wave-uniform: keep them in scalar registers
  const int nt = __builtin_amdgcn_readfirstlane((L % width) / gsz);
  const int g = __builtin_amdgcn_readfirstlane(find_group(t_pre, G, mt));
  const int row0 = __builtin_amdgcn_readfirstlane(t_start[g] + (mt - t_pre[g]) * BM);
  const int rows = __builtin_amdgcn_readfirstlane(min(BM, t_end[g] - row0));

  // ---- buffer resources: the tile's activation rows and the expert's codes
  const BufRsrc ra = make_rsrc(aq + (size_t)row0 * K, (uint32_t)rows * (uint32_t)K);
  const BufRsrc rb = make_rsrc(codes + (size_t)g * K * N, (uint32_t)K * (uint32_t)N);
  uint32_t va[8];                      // activation chunk offsets (step 0)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * (8 * wave + j) + (lane >> 3);
    const int c = (lane & 7) ^ a_key(r);
    va[j] = (uint32_t)min(r, rows - 1) * (uint32_t)K + (uint32_t)(c << 4);
  }
  uint32_t vb[kBLoads];                // weight chunk offsets (step 0)
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    const int kk = kBRowsPerLoad * (kBLoads * wave + j) + lane / kBChunksRow;
    const int c = (lane % kBChunksRow) ^ b_key<BN>(kk);
    int col;
    if (SWIGLU) col = (c < 8) ? nt * (BN / 2) + (c << 4) : I + nt * (BN / 2) + ((c - 8) << 4);
    else col = nt * BN + (c << 4);
    vb[j] = (uint32_t)kk * (uint32_t)N + (uint32_t)col;
  }
  const uint32_t b_step = (uint32_t)BK * (uint32_t)N;

  // ---- per-lane LDS read offsets of the MFMA operands
  int a_rd[8][2];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int r = wm * 128 + f * 16 + (lane & 15);
    const int c0 = (lane >> 4) * 2;
    a_rd[f][0] = a_swz(r, c0);
    a_rd[f][1] = a_swz(r, c0 + 1);
  }
  int b_rd[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int cb;
    if (SWIGLU) cb = (j < 4) ? wn * 64 + j * 16 : 128 + wn * 64 + (j - 4) * 16;
    else cb = wn * (16 * NJ) + j * 16;
    const int Lg = lane & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kk = (lane >> 4) * 32 + 8 * t + (Lg >> 1);
      b_rd[j][t] = BM * BK + b_swz<BN>(kk, cb >> 4) + 8 * (Lg & 1);
    }
  }

  v4f acc[8][NJ];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  auto issue_stage = [&](int ks, int buf) {
    uint8_t* S = smem + buf * kStageBytes;
    const uint32_t sa = (uint32_t)ks * BK, sb = (uint32_t)ks * b_step;
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16(ra, S + (8 * wave + j) * 1024, va[j], sa);
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) dma16(rb, S + BM * BK + (kBLoads * wave + j) * 1024, vb[j], sb);
  };
  auto read_a = [&](int buf, int f) {
    const uint8_t* S = smem + buf * kStageBytes;
    const v4i lo = *reinterpret_cast<const v4i*>(S + a_rd[f][0]);
    const v4i hi = *reinterpret_cast<const v4i*>(S + a_rd[f][1]);
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto read_b = [&](int buf, v8i* bf) {
    const uint8_t* S = smem + buf * kStageBytes;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v2i v = lds_read_tr8(S + b_rd[j][t]);
        bf[j][2 * t] = v[0];
        bf[j][2 * t + 1] = v[1];
      }
  };

  // ---- prologue: stage 0 in LDS, its weight fragments and first activation fragment in registers
  issue_stage(0, 0);
  wait_vmem_all();
  __syncthreads();
  v8i bcur[NJ], bnxt[NJ];
  read_b(0, bcur);
  v8i acur = read_a(0, 0), anxt, a0n = acur;

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) issue_stage(ks + 1, buf ^ 1);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < 7) anxt = read_a(buf, f + 1);
      if (f == 6 && more) {
        // every wave's copy of stage ks+1 has landed: fetch its first fragments
        wait_vmem_all();
        __syncthreads();
        read_b(buf ^ 1, bnxt);
        a0n = read_a(buf ^ 1, 0);
      }
      sched_fence();
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[f][j] = mfma_e4m3_16x16x128(bcur[j], acur, acc[f][j]);
      sched_fence();
      if (f < 7) acur = anxt;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) bcur[j] = bnxt[j];
    acur = a0n;
    __syncthreads();   // stage ks fully consumed before it is refilled
  }

  // ---- epilogue: lane owns row (f*16 + lane%16) and columns cb(j) + 4*(lane/16) + 0..3
  const float* ws = wscale + (size_t)g * N;
  if (SWIGLU) {
    v4f sg[4], su[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cg = nt * (BN / 2) + wn * 64 + j * 16 + 4 * (lane >> 4);
      sg[j] = *reinterpret_cast<const v4f*>(ws + cg);
      su[j] = *reinterpret_cast<const v4f*>(ws + I + cg);
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int ml = wm * 128 + f * 16 + (lane & 15);
      if (ml < rows) {
        const int row = row0 + ml;
        const float sr = ascale[row];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int cg = nt * (BN / 2) + wn * 64 + j * 16 + 4 * (lane >> 4);
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float yg = (acc[f][j][r] * sr) * sg[j][r];
            const float yu = (acc[f][j + 4][r] * sr) * su[j][r];
            o[r] = yg / (1.0f + __expf(-yg)) * yu;
          }
          v2i pk;
          pk[0] = (int)pack_bf16x2(o[0], o[1]);
          pk[1] = (int)pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<v2i*>(out + (size_t)row * I + cg) = pk;
        }
      }
    }
  } else {
    v4f sc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = nt * BN + wn * (16 * NJ) + j * 16 + 4 * (lane >> 4);
      sc[j] = *reinterpret_cast<const v4f*>(ws + c);
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int ml = wm * 128 + f * 16 + (lane & 15);
      if (ml < rows) {
        const int row = row0 + ml;
        const float sr = ascale[row];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int c = nt * BN + wn * (16 * NJ) + j * 16 + 4 * (lane >> 4);
          v2i pk;
          pk[0] = (int)pack_bf16x2((acc[f][j][0] * sr) * sc[j][0], (acc[f][j][1] * sr) * sc[j][1]);
          pk[1] = (int)pack_bf16x2((acc[f][j][2] * sr) * sc[j][2], (acc[f][j][3] * sr) * sc[j][3]);
          *reinterpret_cast<v2i*>(out + (size_t)row * N + c) = pk;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gmm_fp8_fwd(const uint8_t* aq, const float* ascale, const uint8_t* codes, const float* wscale,
                              const int* group_sizes, int G, int M, int K, int N, bool swiglu, uint16_t* out,
                              int* status, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const long long max_m_tiles = (M + BM - 1) / BM + G;
  const size_t table = sizeof(int) * (3 * (size_t)G + 1);
  if (swiglu) {
    const long long grid = max_m_tiles * ((N / 2) / 128);
    hipLaunchKernelGGL((gmm_fp8_fwd_kernel<true, 8>), dim3((unsigned)grid), dim3(kThreads), lds_main<256>() + table,
                       stream, aq, ascale, codes, wscale, group_sizes, G, M, K, N, out, status);
  } else if (N % 256 == 0) {
    const long long grid = max_m_tiles * (N / 256);
    hipLaunchKernelGGL((gmm_fp8_fwd_kernel<false, 8>), dim3((unsigned)grid), dim3(kThreads), lds_main<256>() + table,
                       stream, aq, ascale, codes, wscale, group_sizes, G, M, K, N, out, status);
  } else {
    const long long grid = max_m_tiles * (N / 128);
    hipLaunchKernelGGL((gmm_fp8_fwd_kernel<false, 4>), dim3((unsigned)grid), dim3(kThreads), lds_main<128>() + table,
                       stream, aq, ascale, codes, wscale, group_sizes, G, M, K, N, out, status);
  }
  return hipGetLastError();
}

}  // namespace fp8gmm

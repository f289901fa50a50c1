// Weight-gradient tgmm with in-kernel operand quantization ("MoE fp8
// backward: in-kernel drhs operand quantization + configurable gradient
// dtype", What: the drhs tgmm's operands are quantized inside the kernel, per
// gm-tile and per channel, touching only tiles covered by group_sizes, so no
// reduction ever reads past the valid rows; the gradient uses e5m2 or e4m3).
//
// drhs[g] = sum over non-empty pairs p = (g, t) of
//           (sL_p x sD_p) (.) ( sum_{r in rows(p)} dec(qL[r, :])^T dec(qD[r, :]) )
// with tiles t aligned to the buffer (rows [t*tile_m, (t+1)*tile_m)) and
// intersected with expert g, per-channel scales sL_p = f32(max(amax,1e-12)/448),
// sD_p = f32(max(amax,1e-12)/FMAX_grad), qL = e4m3(lhs/sL), qD = grad(dout/sD).
//
// Two kernels:
//  1. prep: one block per (pair, 64-column chunk of lhs or dout) reads only
//     the pair's valid rows once, reduces the column amax (wave shuffles +
//     LDS), writes the scales, quantizes, and stores the exactly decoded
//     8-bit values as bf16 transposed ([column][row], row-padded with zeros to
//     a multiple of 64) into the workspace.
//  2. gemm: one block per (expert, 256-row k tile, 128-column n tile) walks
//     the expert's pairs; the contraction over rows runs on bf16 MFMA (every
//     e4m3/e5m2 value is exact in bf16 and products are exact in f32), so the
//     sums keep f32 accuracy (gfx950's FP8 MFMA adds its 128 products in a
//     narrower adder, about 2^-16 of the absolute sum, too coarse for an f32
//     gradient).  A per-pair partial accumulator is rescaled by sL x sD and
//     added to the total at each pair boundary.  Experts without rows get
//     zeros.  The f32 output is written with 16-byte streaming stores.
#include "common.hpp"
#include "launch.hpp"

namespace fp8gmm {
namespace {

constexpr int kTileM = 512;       // rows per gm-tile (the only supported value)
constexpr int kPrepCols = 64;     // columns per prep block
constexpr int kChunk = 64;        // contraction rows per GEMM stage
constexpr int kThreads = 256;
constexpr int kLdsStride = kTileM + 8;   // bf16 elements per transposed LDS row (prep)

// Pair table from group_sizes, built by wave 0 into LDS: for pair p (in
// (expert, tile) order) its expert, first row and row count; returns via
// p_base[g] the first pair of expert g (exclusive prefix, p_base[G] = total).
struct PairTable {
  int* g_start;   // [G]
  int* g_end;     // [G]
  int* p_base;    // [G + 1]
};

__device__ __forceinline__ void build_pair_table(const int* __restrict__ group_sizes, int G, int M, PairTable t,
                                                 int* status) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int row_carry = 0, pair_carry = 0, flags = 0;
  for (int base = 0; base < G; base += 64) {
    const int g = base + lane;
    const int raw = g < G ? group_sizes[g] : 0;
    if (raw < 0) flags |= kDevNegativeSize;
    if (raw > M) flags |= kDevSumClamped;
    const int sz = min(max(raw, 0), M);
    const int incl = wave_incl_scan(sz);
    const int e_raw = row_carry + incl;
    const int st = min(e_raw - sz, M), en = min(e_raw, M);
    if (e_raw > M && sz > 0) flags |= kDevSumClamped;
    const int np = en > st ? (en - 1) / kTileM - st / kTileM + 1 : 0;
    const int pincl = wave_incl_scan(np);
    if (g < G) {
      t.g_start[g] = st;
      t.g_end[g] = en;
      t.p_base[g] = pair_carry + pincl - np;
    }
    row_carry = min(__shfl(e_raw, 63, 64), M);
    pair_carry += __shfl(pincl, 63, 64);
  }
  if (lane == 0) t.p_base[G] = pair_carry;
  int any = flags;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) any |= __shfl_xor(any, o, 64);
  if (status != nullptr && lane == 0 && blockIdx.x == 0 && blockIdx.y == 0 && any) atomicOr(status, any);
}

// Rows [r0, r1) of pair p (its expert is g).
__device__ __forceinline__ void pair_rows(const PairTable& t, int g, int p, int& r0, int& r1) {
  const int s = t.g_start[g], e = t.g_end[g];
  const int tile = s / kTileM + (p - t.p_base[g]);
  r0 = max(s, tile * kTileM);
  r1 = min(e, (tile + 1) * kTileM);
}

__device__ __forceinline__ int pair_group(const PairTable& t, int G, int p) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.p_base[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------ prep

template <bool GRAD_E5M2>
__global__ __launch_bounds__(kThreads) void tgmm_prep_kernel(const uint16_t* __restrict__ lhs,
                                                             const uint16_t* __restrict__ dout,
                                                             const int* __restrict__ group_sizes, int G, int M,
                                                             int K, int N, uint16_t* __restrict__ lt,
                                                             uint16_t* __restrict__ dt, float* __restrict__ sl,
                                                             float* __restrict__ sd, int* status) {
  __shared__ int g_start[kMaxGroups], g_end[kMaxGroups], p_base[kMaxGroups + 1];
  __shared__ float red[4][kPrepCols];
  __shared__ __attribute__((aligned(16))) uint16_t tile[kPrepCols * kLdsStride];
  PairTable pt{g_start, g_end, p_base};
  build_pair_table(group_sizes, G, M, pt, blockIdx.y == 0 ? status : nullptr);
  __syncthreads();
  const int p = blockIdx.x;
  if (p >= p_base[G]) return;
  const int g = pair_group(pt, G, p);
  int r0, r1;
  pair_rows(pt, g, p, r0, r1);
  const int R = r1 - r0;
  const int Rpad = (R + kChunk - 1) / kChunk * kChunk;

  // which operand and columns
  const int kc = K / kPrepCols;
  const bool is_l = (int)blockIdx.y < kc;
  const int cols = is_l ? K : N;
  const int c0 = (is_l ? (int)blockIdx.y : (int)blockIdx.y - kc) * kPrepCols;
  const uint16_t* src = is_l ? lhs : dout;
  const float fmax = is_l ? kE4M3Max : (GRAD_E5M2 ? kE5M2Max : kE4M3Max);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid & 7;          // 8-column group
  const int rr = tid >> 3;         // 0..31
  // ---- load the pair's rows (16 per thread) and reduce the column amax
  v4i x[16];
  float am[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) am[e] = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = rr + 32 * i;
    if (r < R) {
      x[i] = *reinterpret_cast<const v4i*>(src + (size_t)(r0 + r) * cols + c0 + cg * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        am[2 * e] = __builtin_fmaxf(am[2 * e], __builtin_fabsf(bf16_lo((uint32_t)x[i][e])));
        am[2 * e + 1] = __builtin_fmaxf(am[2 * e + 1], __builtin_fabsf(bf16_hi((uint32_t)x[i][e])));
      }
    } else {
      x[i] = (v4i){0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v = am[e];
    v = __builtin_fmaxf(v, __shfl_xor(v, 8, 64));
    v = __builtin_fmaxf(v, __shfl_xor(v, 16, 64));
    v = __builtin_fmaxf(v, __shfl_xor(v, 32, 64));
    am[e] = v;
  }
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = am[e];
  }
  __syncthreads();
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = cg * 8 + e;
    const float a = __builtin_fmaxf(__builtin_fmaxf(red[0][c], red[1][c]), __builtin_fmaxf(red[2][c], red[3][c]));
    s[e] = __builtin_fmaxf(a, kAmaxFloor) / fmax;     // IEEE f32 division
  }
  if (tid < kPrepCols) {
    const float a = __builtin_fmaxf(__builtin_fmaxf(red[0][tid], red[1][tid]),
                                    __builtin_fmaxf(red[2][tid], red[3][tid]));
    float* sdst = is_l ? sl + (size_t)p * K : sd + (size_t)p * N;
    sdst[c0 + tid] = __builtin_fmaxf(a, kAmaxFloor) / fmax;
  }
  // ---- quantize, decode exactly, store transposed as bf16
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = rr + 32 * i;
    if (r < Rpad) {
      float q[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q[2 * e] = bf16_lo((uint32_t)x[i][e]) / s[2 * e];
        q[2 * e + 1] = bf16_hi((uint32_t)x[i][e]) / s[2 * e + 1];
      }
      uint32_t w0, w1;
      v2f d[4];
      if (is_l || !GRAD_E5M2) {
        w0 = cvt_e4m3x4(q[0], q[1], q[2], q[3]);
        w1 = cvt_e4m3x4(q[4], q[5], q[6], q[7]);
        d[0] = dec_e4m3x2<false>(w0); d[1] = dec_e4m3x2<true>(w0);
        d[2] = dec_e4m3x2<false>(w1); d[3] = dec_e4m3x2<true>(w1);
      } else {
        w0 = cvt_e5m2x4(q[0], q[1], q[2], q[3]);
        w1 = cvt_e5m2x4(q[4], q[5], q[6], q[7]);
        d[0] = dec_e5m2x2<false>(w0); d[1] = dec_e5m2x2<true>(w0);
        d[2] = dec_e5m2x2<false>(w1); d[3] = dec_e5m2x2<true>(w1);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // decoded 8-bit values have at most 4 significant bits: the bf16 is the f32's high half
        const float v = (r < R) ? d[e >> 1][e & 1] : 0.0f;
        tile[(cg * 8 + e) * kLdsStride + r] = (uint16_t)(__float_as_uint(v) >> 16);
      }
    }
  }
  __syncthreads();
  // ---- write [64 columns][Rpad rows] to the transposed workspace
  uint16_t* dst = (is_l ? lt + ((size_t)p * K + c0) * kTileM : dt + ((size_t)p * N + c0) * kTileM);
  const int vec_per_col = Rpad / 8;
  for (int v = tid; v < kPrepCols * vec_per_col; v += kThreads) {
    const int c = v / vec_per_col, r = (v % vec_per_col) * 8;
    const v4i val = *reinterpret_cast<const v4i*>(&tile[c * kLdsStride + r]);
    *reinterpret_cast<v4i*>(dst + (size_t)c * kTileM + r) = val;
  }
}

// ------------------------------------------------------------------ gemm

constexpr int BMK = 256;   // k rows of drhs per block
constexpr int BNN = 128;   // n columns per block
constexpr int kRowB = kChunk * 2;                     // 128 bytes per LDS row
constexpr int kStageG = (BMK + BNN) * kRowB;          // 48 KiB
constexpr int kLdsG = 2 * kStageG;

__device__ __forceinline__ int g_swz(int row, int chunk) { return row * kRowB + ((chunk ^ (row & 7)) << 4); }

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void tgmm_gemm_kernel(const uint16_t* __restrict__ lt, const uint16_t* __restrict__ dt,
                      const float* __restrict__ sl, const float* __restrict__ sd,
                      const int* __restrict__ group_sizes, int G, int M, int K, int N,
                      float* __restrict__ drhs) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* g_start = reinterpret_cast<int*>(smem + kLdsG);
  int* g_end = g_start + G;
  int* p_base = g_end + G;
  PairTable pt{g_start, g_end, p_base};
  build_pair_table(group_sizes, G, M, pt, nullptr);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wk = wave >> 1, wn = wave & 1;
  const int kt_n = K / BMK, nt_n = N / BNN;
  // blocks of one expert are adjacent; within it k tiles vary fastest so the
  // 8 XCDs share the dout tile of the same n tile
  const int bid = blockIdx.x;
  const int g = bid / (kt_n * nt_n);
  const int rem = bid % (kt_n * nt_n);
  const int kt = rem % kt_n, nt = rem / kt_n;
  float* out = drhs + ((size_t)g * K + (size_t)kt * BMK) * N + (size_t)nt * BNN;

  v4f tot[8][4];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int p0 = p_base[g], p1 = p_base[g + 1];
  if (p1 > p0) {
    // per-thread load slots: A (lt) 8 x 16 B, B (dt) 4 x 16 B per stage
    int a_off[8], b_off[4];
    size_t a_src[8], b_src[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + kThreads * j;
      const int row = i >> 3, c = i & 7;
      a_src[j] = (size_t)(kt * BMK + row) * kTileM + c * 8;
      a_off[j] = g_swz(row, c);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + kThreads * j;
      const int row = i >> 3, c = i & 7;
      b_src[j] = (size_t)(nt * BNN + row) * kTileM + c * 8;
      b_off[j] = BMK * kRowB + g_swz(row, c);
    }
    int a_rd[8][2], b_rd[4][2];
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int s = 0; s < 2; ++s) a_rd[f][s] = g_swz(wk * 128 + f * 16 + (lane & 15), s * 4 + (lane >> 4));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        b_rd[j][s] = BMK * kRowB + g_swz(wn * 64 + j * 16 + (lane & 15), s * 4 + (lane >> 4));

    v4i sa[8], sb[4];
    // flattened (pair, chunk) sequence of this expert
    auto chunks_of = [&](int p) {
      int r0, r1;
      pair_rows(pt, g, p, r0, r1);
      return (r1 - r0 + kChunk - 1) / kChunk;
    };
    auto load = [&](int p, int c) {
      const uint16_t* lp = lt + (size_t)p * K * kTileM + c * kChunk;
      const uint16_t* dp = dt + (size_t)p * N * kTileM + c * kChunk;
#pragma unroll
      for (int j = 0; j < 8; ++j) sa[j] = *reinterpret_cast<const v4i*>(lp + a_src[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) sb[j] = *reinterpret_cast<const v4i*>(dp + b_src[j]);
    };
    auto store = [&](int buf) {
      uint8_t* S = smem + buf * kStageG;
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<v4i*>(S + a_off[j]) = sa[j];
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(S + b_off[j]) = sb[j];
    };

    int p = p0, c = 0, nc = chunks_of(p0);
    load(p, c);
    store(0);
    __syncthreads();
    int buf = 0;
    v4f part[8][4];
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    while (true) {
      // next (pair, chunk)
      int pn = p, cn = c + 1, ncn = nc;
      if (cn == nc) { pn = p + 1; cn = 0; ncn = pn < p1 ? chunks_of(pn) : 0; }
      const bool more = pn < p1;
      if (more) load(pn, cn);
      const uint8_t* S = smem + buf * kStageG;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v8bf bfr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[j] = *reinterpret_cast<const v8bf*>(S + b_rd[j][s]);
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          const v8bf af = *reinterpret_cast<const v8bf*>(S + a_rd[f][s]);
#pragma unroll
          for (int j = 0; j < 4; ++j) part[f][j] = mfma_bf16_16x16x32(bfr[j], af, part[f][j]);
        }
      }
      if (cn == 0) {
        // pair p complete: total += partial * sL[k] * sD[n]
        const float* slp = sl + (size_t)p * K + kt * BMK + wk * 128 + (lane & 15);
        const float* sdp = sd + (size_t)p * N + nt * BNN + wn * 64 + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f dsc = *reinterpret_cast<const v4f*>(sdp + j * 16);
#pragma unroll
          for (int f = 0; f < 8; ++f) {
            const float lsc = slp[f * 16];
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[f][j][r] += (part[f][j][r] * lsc) * dsc[r];
            part[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
          }
        }
      }
      if (!more) break;
      store(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      p = pn; c = cn; nc = ncn;
    }
  }
  // ---- store: lane owns k = wk*128 + f*16 + lane%16, n = wn*64 + j*16 + 4*(lane/16) + 0..3
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    float* orow = out + (size_t)(wk * 128 + f * 16 + (lane & 15)) * N + wn * 64 + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(tot[f][j], reinterpret_cast<v4f*>(orow + j * 16));
  }
}

}  // namespace

size_t tgmm_workspace_bytes(long long M, long long K, long long N, int G) {
  const long long tmax = (M + kTileM - 1) / kTileM + G - 1;
  if (tmax <= 0) return 0;
  const size_t a = 256;
  auto al = [&](size_t x) { return (x + a - 1) / a * a; };
  return al((size_t)tmax * K * kTileM * 2) + al((size_t)tmax * N * kTileM * 2) + al((size_t)tmax * K * 4) +
         al((size_t)tmax * N * 4);
}

hipError_t launch_tgmm_quant(const uint16_t* lhs, const uint16_t* dout, const int* group_sizes, int G, int M, int K,
                             int N, bool grad_e5m2, float* drhs, float* dbg_sl, float* dbg_sd, void* ws,
                             int* status, hipStream_t stream) {
  const long long tmax = (M + kTileM - 1) / kTileM + G - 1;
  const size_t a = 256;
  auto al = [&](size_t x) { return (x + a - 1) / a * a; };
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint16_t* lt = reinterpret_cast<uint16_t*>(base);
  uint16_t* dt = reinterpret_cast<uint16_t*>(base + al((size_t)tmax * K * kTileM * 2));
  float* sl = reinterpret_cast<float*>(base + al((size_t)tmax * K * kTileM * 2) + al((size_t)tmax * N * kTileM * 2));
  float* sd = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(sl) + al((size_t)tmax * K * 4));
  if (dbg_sl) sl = dbg_sl;
  if (dbg_sd) sd = dbg_sd;
  if (tmax > 0 && M > 0) {
    dim3 grid((unsigned)tmax, (unsigned)(K / kPrepCols + N / kPrepCols));
    if (grad_e5m2)
      hipLaunchKernelGGL(tgmm_prep_kernel<true>, grid, dim3(kThreads), 0, stream, lhs, dout, group_sizes, G, M, K,
                         N, lt, dt, sl, sd, status);
    else
      hipLaunchKernelGGL(tgmm_prep_kernel<false>, grid, dim3(kThreads), 0, stream, lhs, dout, group_sizes, G, M, K,
                         N, lt, dt, sl, sd, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t lds = kLdsG + sizeof(int) * (3 * (size_t)G + 1);
  hipLaunchKernelGGL(tgmm_gemm_kernel, dim3((unsigned)((long long)G * (K / BMK) * (N / BNN))), dim3(kThreads), lds,
                     stream, lt, dt, sl, sd, group_sizes, G, M, K, N, drhs);
  return hipGetLastError();
}

}  // namespace fp8gmm

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
//     LDS), writes the scales and stores the 8-bit codes row-major into the
//     pair's slab of the workspace ([512 rows][columns], rows past the pair's
//     end up to the next multiple of 32 hold zero codes).  One block of it
//     also computes the GEMM's item deal (build_item_schedule) meanwhile.
//  2. gemm: persistent, walking each block's share of the work items
//     (expert, k tile of 256 rows -- 128 when K is not a multiple of 256 --,
//     128-column n tile), dealt so that the blocks' modelled loads stay even;
//     an item covers the expert's pairs 128 (64) rows at a time.  The code chunks of both operands are copied HBM -> LDS by
//     buffer loads with an LDS destination through a three- (four-) stage
//     ring that runs across pairs and items, so copy latency is
//     paid once per block rather than once per tile; a pair's last stage
//     reads zeros past its padded rows (the copy's buffer range ends there).  The contraction runs
//     over rows, which is the slow axis of both tiles, so the MFMA operands
//     are read with the transposing ds_read_tr8_b64 (8 consecutive rows of
//     one column per lane) and widened to bf16 exactly.  bf16 MFMA (every
//     e4m3/e5m2 value is exact in bf16 and products are exact in f32) keeps
//     f32 accuracy; gfx950's FP8 MFMA adds its 128 products in a narrower
//     adder, about 2^-16 of the absolute sum, too coarse for an f32 gradient.
//     Eight (four) waves own 64 x 64 of the tile each, two per SIMD (the
//     128-row form runs two blocks per CU); a per-pair
//     partial accumulator is rescaled by sL x sD and added to the total at
//     the pair's end.  The pair's scales travel with each stage's copy into
//     the ring, so the rescale reads LDS and never waits on a global load
//     (such a wait also waits for every copy in flight).  A pair's last
//     stage runs only the 32-row sub-steps its rows cover.  Experts without
//     rows get zeros.  The f32 output is written with 16-byte streaming
//     stores of whole cache lines.
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace fp8gmm {
namespace {

constexpr int kTileM = 512;       // rows per gm-tile (the only supported value)
constexpr int kPrepCols = 64;     // columns per prep block
constexpr int kSub = 32;          // contraction rows per MFMA sub-step (slabs are padded to this)
constexpr int kThreads = 256;

// Pair table from group_sizes, built by wave 0 into LDS: expert g owns rows
// [g_start[g], g_start[g + 1]) (clamped to the buffer) and pairs
// [p_base[g], p_base[g + 1]) in (expert, tile) order.
struct PairTable {
  int* g_start;   // [G + 1]
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
      t.p_base[g] = pair_carry + pincl - np;
    }
    if (g == G - 1) t.g_start[G] = en;   // the next expert would start here
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
  const int s = t.g_start[g], e = t.g_start[g + 1];
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

// Item deal of the GEMM (tgmm_gemm_kernel): expert g's work item j goes to
// block (o_g + j) mod nb.  Every block gets per_g / nb items of each expert,
// and the per_g mod nb that remain go to nb-consecutive (cyclic) blocks from
// o_g.  Plain round-robin over the item index (o_g = g * per_g mod nb) lets
// the blocks that draw the heavy experts' remainders run ~6 % longer than
// the mean on a Zipf routing; here the experts are taken by decreasing cost
// and each one's remainder starts at the least-loaded window so far, which
// brings the modelled max/mean to within 1 % (measured with per-wave timers
// on 32 experts, 19661 Zipf-routed rows, 7168 x 2048: the slowest block 1.5 %
// above the mean, against 5.5 % for round-robin).  The cost of an item is a model
// of the GEMM's time per item from per-wave timers (ticks per 32-row sub-step,
// per ring stage, per pair-end rescale and per tile store).
constexpr int kMaxSchedGroups = 256;   // larger G keeps the round-robin deal
constexpr int kMaxSchedBlocks = 512;   // the GEMM's grid: one or two blocks per CU
constexpr int kCostSub = 730, kCostStage = 1300, kCostPair = 1100, kCostItem = 5930;

// Run by every thread of one block (blockDim.x >= 64, a multiple of 64) after
// the pair table is in LDS; writes sched[g] = o_g for every expert.
__device__ void build_item_schedule(const PairTable& pt, int G, int chunk, int per_g, int nb,
                                    int* __restrict__ sched) {
  __shared__ int s_cost[kMaxSchedGroups], s_order[kMaxSchedGroups];
  __shared__ int s_pre[kMaxSchedBlocks + 1];   // s_pre[t]: load of blocks [0, t) from the remainders dealt so far
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int g = tid; g < G; g += nt) {
    int c = kCostItem;
    for (int p = pt.p_base[g]; p < pt.p_base[g + 1]; ++p) {
      int r0, r1;
      pair_rows(pt, g, p, r0, r1);
      const int sub = (r1 - r0 + kSub - 1) / kSub;
      c += kCostSub * sub + kCostStage * ((sub * kSub + chunk - 1) / chunk) + kCostPair;
    }
    s_cost[g] = (c + 255) >> 8;   // units of 256 ticks: the prefix sums stay within 32 bits
  }
  for (int t = tid; t <= nb; t += nt) s_pre[t] = 0;
  __syncthreads();
  for (int g = tid; g < G; g += nt) {   // rank by decreasing cost, ties by expert index
    const int c = s_cost[g];
    int r = 0;
    for (int h = 0; h < G; ++h) {
      const int ch = s_cost[h];
      r += (ch > c) || (ch == c && h < g);
    }
    s_order[r] = g;
  }
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid, extra = per_g % nb, per_lane = (nb + 63) / 64, t0 = lane * per_lane;
  for (int i = 0; i < G; ++i) {
    const int g = s_order[i];
    int bo = 0;
    if (extra != 0) {
      // the window [o, o + extra) (cyclic) with the smallest load; the smallest o on ties
      int best = 0x7fffffff;
      const int tot = s_pre[nb];
      for (int k = 0; k < per_lane; ++k) {
        const int o = t0 + k;
        if (o < nb) {
          const int e = o + extra;
          const int w = e <= nb ? s_pre[e] - s_pre[o] : tot - s_pre[o] + s_pre[e - nb];
          if (w < best) {
            best = w;
            bo = o;
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const int wb = __shfl_xor(best, off, 64), ob = __shfl_xor(bo, off, 64);
        if (wb < best || (wb == best && ob < bo)) {
          best = wb;
          bo = ob;
        }
      }
      // add the expert's cost to the window's blocks: s_pre[t] += c * |window intersect [0, t)|
      // (lane L owns entries [L * per_lane, (L + 1) * per_lane) up to nb; lane 63 also owns nb when
      // the lanes' ranges end exactly there)
      const int c = s_cost[g], end = bo + extra;
      auto add = [&](int t) {
        const int n = end <= nb ? min(max(t - bo, 0), extra) : min(max(t - bo, 0), nb - bo) + min(t, end - nb);
        s_pre[t] += c * n;
      };
      for (int k = 0; k < per_lane; ++k)
        if (t0 + k <= nb) add(t0 + k);
      if (lane == 63 && 64 * per_lane == nb) add(nb);
    }
    if (lane == 0) sched[g] = bo;
  }
}

// ------------------------------------------------------------------ prep

template <bool GRAD_E5M2>
__global__ __launch_bounds__(kThreads) void tgmm_prep_kernel(const uint16_t* __restrict__ lhs,
                                                             const uint16_t* __restrict__ dout,
                                                             const int* __restrict__ group_sizes, int G, int M,
                                                             int K, int N, uint8_t* __restrict__ ql,
                                                             uint8_t* __restrict__ qd, float* __restrict__ sl,
                                                             float* __restrict__ sd, int* status, int* sched,
                                                             int s_chunk, int s_per_g, int s_nb) {
  __shared__ int g_start[kMaxGroups + 1], p_base[kMaxGroups + 1];
  __shared__ float red[4][kPrepCols];
  PairTable pt{g_start, p_base};
  // blockIdx.x = 64-column chunk (fastest, so that blocks dispatched together
  // read neighbouring strips of the same rows), blockIdx.y = pair
  build_pair_table(group_sizes, G, M, pt, blockIdx.x == 0 ? status : nullptr);
  __syncthreads();
  // the GEMM's item deal, by one block while the others quantize
  if (sched != nullptr && blockIdx.x == 0 && blockIdx.y == 0) build_item_schedule(pt, G, s_chunk, s_per_g, s_nb, sched);
  const int p = blockIdx.y;
  if (p >= p_base[G]) return;
  const int g = pair_group(pt, G, p);
  int r0, r1;
  pair_rows(pt, g, p, r0, r1);
  const int R = r1 - r0;
  const int Rpad = (R + kSub - 1) / kSub * kSub;

  // which operand and columns
  const int kc = K / kPrepCols;
  const bool is_l = (int)blockIdx.x < kc;
  const int cols = is_l ? K : N;
  const int c0 = (is_l ? (int)blockIdx.x : (int)blockIdx.x - kc) * kPrepCols;
  const uint16_t* src = is_l ? lhs : dout;
  const float fmax = is_l ? kE4M3Max : (GRAD_E5M2 ? kE5M2Max : kE4M3Max);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid & 7;          // 8-column group
  const int rr = tid >> 3;         // 0..31
  // ---- load the pair's rows (16 per thread) and reduce the column amax.
  // Every load goes out before any is used: a row group past the pair's rows
  // is skipped by a wave-uniform branch, and the rows of the last group past
  // the pair's end read zeros through a buffer range that ends there.
  const BufRsrc rsrc = make_rsrc(src + (size_t)r0 * cols, (uint32_t)R * (uint32_t)cols * 2u);
  const int n_it = (R + 31) / 32;
  v4i x[16];
  float am[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) am[e] = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < n_it)
      x[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                         rsrc, (uint32_t)((rr + 32 * i) * cols + c0 + cg * 8) * 2u, 0u, kCpolStream));
    else
      x[i] = (v4i){0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      am[2 * e] = __builtin_fmaxf(am[2 * e], __builtin_fabsf(bf16_lo((uint32_t)x[i][e])));
      am[2 * e + 1] = __builtin_fmaxf(am[2 * e + 1], __builtin_fabsf(bf16_hi((uint32_t)x[i][e])));
    }
  }
  // the quantize pass widens the raw rows again instead of keeping these f32 values
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(x[i]));
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
  // ---- quantize (f32 quotient, saturating RNE) and store the codes row-major in the pair's slab.
  // The quotient comes from the column's reciprocal (div_by_scale); a lane
  // with a non-finite scale (an Inf in its columns) divides directly.
  float rs[8];
  bool finite = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    rs[e] = 1.0f / s[e];
    finite = finite && __builtin_isfinite(s[e]);
  }
  uint8_t* dst = (is_l ? ql + (size_t)p * kTileM * K : qd + (size_t)p * kTileM * N) + c0 + cg * 8;
  auto quantize = [&](auto fast_c) {
    constexpr bool FAST = decltype(fast_c)::value;
    auto quo = [&](float v, int e) { return FAST ? div_by_scale(v, s[e], rs[e]) : v / s[e]; };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rr + 32 * i;
      if (r < Rpad) {
        float q[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          q[2 * e] = quo(bf16_lo((uint32_t)x[i][e]), 2 * e);
          q[2 * e + 1] = quo(bf16_hi((uint32_t)x[i][e]), 2 * e + 1);
        }
        v2i w;
        if (is_l || !GRAD_E5M2) {
          w[0] = (int)cvt_e4m3x4(q[0], q[1], q[2], q[3]);
          w[1] = (int)cvt_e4m3x4(q[4], q[5], q[6], q[7]);
        } else {
          w[0] = (int)cvt_e5m2x4(q[0], q[1], q[2], q[3]);
          w[1] = (int)cvt_e5m2x4(q[4], q[5], q[6], q[7]);
        }
        if (r >= R) w = (v2i){0, 0};
        *reinterpret_cast<v2i*>(dst + (size_t)r * cols) = w;
      }
    }
  };
  if (finite) quantize(std::true_type{});
  else quantize(std::false_type{});
}

// ------------------------------------------------------------------ buffer-wide baseline
//
// The backward quantization the in-kernel path replaces ("MoE fp8 backward:
// in-kernel drhs operand quantization + configurable gradient dtype", What:
// lhs rows quantized again with one scale each, that scale folded into the
// gradient, one gradient scale per column, all over the static buffer, so an
// Inf in a stale row reaches a column scale and the gradient becomes NaN).  Every row of the
// buffer is read, stale rows included; the contraction then reuses the GEMM
// below with per-pair scales 1 (lhs) and the column scale (gradient).

constexpr int kDenseRows = 128;   // rows per block of the column passes
constexpr int kDenseCols = 2048;  // columns per block (8 per thread)

// partial[rc][n] = max over the rows of chunk rc of |f32(dout[r,n] * srow[r])| (maxNum)
__global__ __launch_bounds__(256) void dense_colmax_kernel(const uint16_t* __restrict__ dout,
                                                           const float* __restrict__ srow, int M, int N,
                                                           float* __restrict__ partial) {
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= N) return;
  const int r0 = blockIdx.x * kDenseRows, r1 = min(M, r0 + kDenseRows);
  float am[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) am[e] = 0.f;
#pragma unroll 4
  for (int r = r0; r < r1; ++r) {
    const v4i x = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(dout + (size_t)r * N + c));
    const float s = srow[r];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      am[2 * e] = __builtin_fmaxf(am[2 * e], __builtin_fabsf(bf16_lo((uint32_t)x[e]) * s));
      am[2 * e + 1] = __builtin_fmaxf(am[2 * e + 1], __builtin_fabsf(bf16_hi((uint32_t)x[e]) * s));
    }
  }
  float* dst = partial + (size_t)blockIdx.x * N + c;
  *reinterpret_cast<v4f*>(dst) = (v4f){am[0], am[1], am[2], am[3]};
  *reinterpret_cast<v4f*>(dst + 4) = (v4f){am[4], am[5], am[6], am[7]};
}

// scol[n] = f32(max(amax, 1e-12) / fmax) over the chunk maxima: a block takes
// 32 columns, its eight 32-thread groups stride over the chunks, LDS combines.
__global__ __launch_bounds__(256) void dense_colscale_kernel(const float* __restrict__ partial, int RC, int N,
                                                             float fmax, float* __restrict__ scol) {
  __shared__ float red[8][32];
  const int c = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int n = blockIdx.x * 32 + c;
  float a = 0.f;
  if (n < N)
    for (int rc = grp; rc < RC; rc += 8) a = __builtin_fmaxf(a, partial[(size_t)rc * N + n]);
  red[grp][c] = a;
  __syncthreads();
  if (grp == 0 && n < N) {
#pragma unroll
    for (int i = 1; i < 8; ++i) a = __builtin_fmaxf(a, red[i][c]);
    scol[n] = __builtin_fmaxf(a, kAmaxFloor) / fmax;
  }
}

// qD[r, n] = grad( f32( f32(dout[r,n] * srow[r]) / scol[n] ) ) for every row of the buffer
template <bool GRAD_E5M2>
__global__ __launch_bounds__(256) void dense_quant_kernel(const uint16_t* __restrict__ dout,
                                                          const float* __restrict__ srow,
                                                          const float* __restrict__ scol, int M, int N,
                                                          uint8_t* __restrict__ qD) {
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= N) return;
  const int r0 = blockIdx.x * kDenseRows, r1 = min(M, r0 + kDenseRows);
  const v4f sa = *reinterpret_cast<const v4f*>(scol + c), sb = *reinterpret_cast<const v4f*>(scol + c + 4);
  const float sc[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
#pragma unroll 4
  for (int r = r0; r < r1; ++r) {
    const v4i x = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(dout + (size_t)r * N + c));
    const float s = srow[r];
    float q[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[2 * e] = (bf16_lo((uint32_t)x[e]) * s) / sc[2 * e];
      q[2 * e + 1] = (bf16_hi((uint32_t)x[e]) * s) / sc[2 * e + 1];
    }
    v2i w;
    if (GRAD_E5M2) {
      w[0] = (int)cvt_e5m2x4(q[0], q[1], q[2], q[3]);
      w[1] = (int)cvt_e5m2x4(q[4], q[5], q[6], q[7]);
    } else {
      w[0] = (int)cvt_e4m3x4(q[0], q[1], q[2], q[3]);
      w[1] = (int)cvt_e4m3x4(q[4], q[5], q[6], q[7]);
    }
    *reinterpret_cast<v2i*>(qD + (size_t)r * N + c) = w;
  }
}

// The valid rows' codes of the buffer-wide operands into the GEMM's pair
// slabs (zeros up to the next 32 rows), with per-pair scales 1 for the lhs
// (its row scales are inside the gradient) and scol for the gradient.
__global__ __launch_bounds__(kThreads) void dense_gather_kernel(const uint8_t* __restrict__ qLd,
                                                                const uint8_t* __restrict__ qDd,
                                                                const float* __restrict__ scol,
                                                                const int* __restrict__ group_sizes, int G, int M,
                                                                int K, int N, uint8_t* __restrict__ ql,
                                                                uint8_t* __restrict__ qd, float* __restrict__ sl,
                                                                float* __restrict__ sd, int* status, int* sched,
                                                                int s_chunk, int s_per_g, int s_nb) {
  __shared__ int g_start[kMaxGroups + 1], p_base[kMaxGroups + 1];
  PairTable pt{g_start, p_base};
  build_pair_table(group_sizes, G, M, pt, blockIdx.y == 0 ? status : nullptr);
  __syncthreads();
  if (sched != nullptr && blockIdx.x == 0 && blockIdx.y == 0) build_item_schedule(pt, G, s_chunk, s_per_g, s_nb, sched);
  const int p = blockIdx.x;
  if (p >= p_base[G]) return;
  const int g = pair_group(pt, G, p);
  int r0, r1;
  pair_rows(pt, g, p, r0, r1);
  const int R = r1 - r0;
  const int Rpad = (R + kSub - 1) / kSub * kSub;
  const int kc = K / kPrepCols;
  const bool is_l = (int)blockIdx.y < kc;
  const int cols = is_l ? K : N;
  const int c0 = (is_l ? (int)blockIdx.y : (int)blockIdx.y - kc) * kPrepCols;
  const int tid = threadIdx.x, cg = tid & 7, rr = tid >> 3;
  const uint8_t* src = (is_l ? qLd : qDd) + c0 + cg * 8;
  uint8_t* dst = (is_l ? ql + (size_t)p * kTileM * K : qd + (size_t)p * kTileM * N) + c0 + cg * 8;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = rr + 32 * i;
    if (r < Rpad) {
      v2i w = (v2i){0, 0};
      if (r < R) w = *reinterpret_cast<const v2i*>(src + (size_t)(r0 + r) * cols);
      *reinterpret_cast<v2i*>(dst + (size_t)r * cols) = w;
    }
  }
  if (tid < kPrepCols) {
    if (is_l) sl[(size_t)p * K + c0 + tid] = 1.0f;
    else sd[(size_t)p * N + c0 + tid] = scol[c0 + tid];
  }
}

// ------------------------------------------------------------------ gemm

// Two geometries of the GEMM, by the width of the k tile (drhs rows per work
// item), BMK = 256 when K allows it, else 128:
//   256: 8 waves (4 along k x 2 along n, 64 x 64 each), 128-row stages in a
//        three-slot ring (144 KB), one block per CU;
//   128: 4 waves (2 x 2), 64-row stages in a four-slot ring (68 KB), two
//        blocks per CU.
// Measured on the dropless 7168 x 2048 gradient (K = 7168 takes the 256 form):
// the GEMM ran 911 us with 256-row k tiles against 939 us with 128-row tiles
// and two blocks per CU (its MFMAs busy 28 % of the time, waves stalled on
// the vector-memory counter 45 %: the copies' latency, not bandwidth, bounds
// both forms).
template <int BMK_>
struct TgCfg {
  static constexpr int BMK = BMK_;                 // drhs rows (k) per work item
  static constexpr int BNN = 128;                  // drhs columns (n) per work item
  static constexpr bool kWide = BMK_ == 256;
  static constexpr int kThreads = kWide ? 512 : 256;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kChunk = kWide ? 128 : 64;  // contraction rows per stage (sub-steps of kSub)
  static constexpr int kStages = kWide ? 3 : 4;
  static constexpr int kBlocksPerCU = kWide ? 1 : 2;
  static constexpr int kAStage = kChunk * BMK;     // qL codes [kChunk rows][BMK k]
  static constexpr int kBStage = kChunk * BNN;     // qD codes [kChunk rows][128 n]
  static constexpr int kSStage = 4 * (BMK + BNN);  // the stage's pair's scales: sL [BMK k], sD [128 n]
  static constexpr int kStage = kAStage + kBStage + kSStage;
  static constexpr int kLds = kStages * kStage;
  static constexpr int kALoads = kAStage / (kWaves * 1024);   // 1 KB wave-wide loads per wave per stage
  static constexpr int kBLoads = kBStage / (kWaves * 1024);
  static constexpr int kLoads = kALoads + kBLoads + 1;        // + one 256-byte scale slice per wave
  static constexpr int kARows = 1024 / BMK;                   // qL rows per 1 KB load
  static constexpr int kAChunks = BMK / 16;                   // 16-byte chunks per qL row
  static constexpr int kSlicesL = BMK / 64;                   // 256-byte sL slices per stage
  static_assert(kBlocksPerCU * (kLds + sizeof(int) * 2 * (kMaxGroups + 1) + sizeof(uint16_t) * kMaxGroups) <=
                    160 * 1024,
                "the rings, expert tables and item offsets of a CU's blocks fit the LDS");
  static_assert(kLoads * (kStages - 1) < 64, "outstanding copies fit vmcnt");
  // 16-byte chunk swizzles: the 16 lanes of a transposing read touch 8
  // consecutive rows at one chunk, and two such groups are served together.
  static __device__ __forceinline__ int a_key(int row) { return kWide ? (row & 15) : ((row >> 1) & 7); }
  static __device__ __forceinline__ int l_slot(int row, int chunk) { return row * BMK + ((chunk ^ a_key(row)) << 4); }
  static __device__ __forceinline__ int d_slot(int row, int chunk) { return row * BNN + ((chunk ^ ((row >> 1) & 7)) << 4); }
};

// 8 codes (8 consecutive rows of one column) -> 8 bf16, exactly.
template <bool E5M2>
__device__ __forceinline__ v4i widen8(const v2i& c) {
  v4i o;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    v2bf lo, hi;
    if (E5M2) {
      lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(c[d], 1.0f, false);
      hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(c[d], 1.0f, true);
    } else {
      lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[d], 1.0f, false);
      hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[d], 1.0f, true);
    }
    o[2 * d] = __builtin_bit_cast(int, lo);
    o[2 * d + 1] = __builtin_bit_cast(int, hi);
  }
  return o;
}

// Where a wave's share of a stage's copy goes: operand codes (kALoads +
// kBLoads 1 KB loads) and one 256-byte slice of the pair's scales (the first
// kSlicesL waves the sL slices, the next two the sD halves, any further waves
// the sD halves again, landing on the same bytes with the same values), so
// every wave issues the same number of copies per stage.
template <class C>
struct StageCopy {
  BufRsrc ra, rb, rs;
  uint32_t va[C::kALoads], vb[C::kBLoads];   // per-lane offsets (held by value: no array in memory)
  uint32_t soa, sob, vs, s_lds;
};

// One stage of kChunk rows: optionally start the copy of a later stage into `wr`,
// then read this stage's operands from `rd` and run its first `nsub` (of NS)
// 32-row sub-steps of 16 MFMAs per wave.  On a pair's last stage (`last`)
// the partial is rescaled by the pair's scales, read from this stage's slot,
// and added to the total.
// `wr` and `rd` are distinct ring slots; marking them __restrict__ lets the
// compiler see that the reads cannot depend on the copy just issued, so it
// adds no wait for it (the kernel's own wait + barrier order the ring).
template <bool GRAD_E5M2, class C, int NS = C::kChunk / kSub>
__device__ __forceinline__ void tgmm_stage(uint8_t* __restrict__ wr, const uint8_t* __restrict__ rd, bool copy,
                                           const StageCopy<C>& cp, int wave, const int* a_rd, const int* b_rd,
                                           int nsub, bool last, int sl_rd, int sd_rd, v4f (&part)[4][4],
                                           v4f (&tot)[4][4]) {
  // The copy of a later stage is spread over the sub-steps (copy q goes out
  // at the top of sub-step q * NS / kLoads): issued all at once, the eight
  // waves' 56 copies queue behind each other in the CU's address unit and the
  // last waves wait there for most of a sub-step before their first MFMA.
  auto issue_copy = [&](int q) __attribute__((always_inline)) {
    if (q < C::kALoads) {
      dma16(cp.ra, wr + (C::kALoads * wave + q) * 1024, cp.va[q], cp.soa);
    } else if (q < C::kALoads + C::kBLoads) {
      const int j = q - C::kALoads;
      dma16(cp.rb, wr + C::kAStage + (C::kBLoads * wave + j) * 1024, cp.vb[j], cp.sob);
    } else {
      dma4(cp.rs, wr + C::kAStage + C::kBStage + cp.s_lds, cp.vs, 0);
    }
  };
  // Sub-steps are software-pipelined: the codes of sub-step s+1 are read
  // before sub-step s's MFMAs and widened after them.
  v4i bo[4], ao[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bo[j] = widen8<GRAD_E5M2>(lds_read_tr8(rd + b_rd[j]));
#pragma unroll
  for (int f = 0; f < 4; ++f) ao[f] = widen8<false>(lds_read_tr8(rd + a_rd[f]));
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s >= nsub) break;     // a pair's last stage: rows past its 32-row padding are not computed
    prio_by_progress(s);
    if (copy) {
#pragma unroll
      for (int q = 0; q < C::kLoads; ++q)
        if (q * NS / C::kLoads == s) issue_copy(q);
    }
    v2i cb[4], ca[4];
    if (s + 1 < NS) {
#pragma unroll
      for (int j = 0; j < 4; ++j) cb[j] = lds_read_tr8(rd + b_rd[j] + (s + 1) * 32 * C::BNN);
#pragma unroll
      for (int f = 0; f < 4; ++f) ca[f] = lds_read_tr8(rd + a_rd[f] + (s + 1) * 32 * C::BMK);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        part[f][j] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, bo[j]), __builtin_bit_cast(v8bf, ao[f]), part[f][j]);
    if (s + 1 < NS) {
#pragma unroll
      for (int j = 0; j < 4; ++j) bo[j] = widen8<GRAD_E5M2>(cb[j]);
#pragma unroll
      for (int f = 0; f < 4; ++f) ao[f] = widen8<false>(ca[f]);
    }
  }
  prio_by_progress<3>();
  if (copy && nsub < NS) {   // the copies of the sub-steps a short stage does not run
#pragma unroll
    for (int q = 0; q < C::kLoads; ++q)
      if (q * NS / C::kLoads >= nsub) issue_copy(q);
  }
  if (last) {
    // pair complete: total += partial * sL[k] * sD[n]
    float slv[4];
    v4f sdv[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) slv[f] = *reinterpret_cast<const float*>(rd + sl_rd + 64 * f);
#pragma unroll
    for (int j = 0; j < 4; ++j) sdv[j] = *reinterpret_cast<const v4f*>(rd + sd_rd + 64 * j);
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[f][j][r] = __builtin_fmaf(part[f][j][r] * slv[f], sdv[j][r], tot[f][j][r]);
        part[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
      }
  }
}

template <bool GRAD_E5M2, int BMK_>
__global__ __attribute__((amdgpu_flat_work_group_size(TgCfg<BMK_>::kThreads, TgCfg<BMK_>::kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void tgmm_gemm_kernel(const uint8_t* __restrict__ ql, const uint8_t* __restrict__ qd,
                      const float* __restrict__ sl, const float* __restrict__ sd,
                      const int* __restrict__ group_sizes, const int* __restrict__ sched, int G, int M, int K,
                      int N, float* __restrict__ drhs) {
  using C = TgCfg<BMK_>;
  constexpr int BMK = C::BMK, BNN = C::BNN, kChunk = C::kChunk, kStagesG = C::kStages, kStageG = C::kStage;
  constexpr int kAStage = C::kAStage, kBStage = C::kBStage, kALoadsG = C::kALoads, kBLoadsG = C::kBLoads;
  constexpr int kLoadsG = C::kLoads;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* g_start = reinterpret_cast<int*>(smem + C::kLds);
  int* p_base = g_start + G + 1;
  uint16_t* i_off = reinterpret_cast<uint16_t*>(p_base + G + 1);   // o_g of the item deal
  PairTable pt{g_start, p_base};
  build_pair_table(group_sizes, G, M, pt, nullptr);
  const int per_g = (K / BMK) * (N / BNN);
  const int nb = gridDim.x;
  for (int g = threadIdx.x; g < G; g += C::kThreads) {
    // reduced mod nb whatever the workspace holds, so every item index stays in range
    int o = sched != nullptr ? sched[g] % nb : (int)((long long)g * per_g % nb);
    i_off[g] = (uint16_t)(o < 0 ? o + nb : o);
  }
  __syncthreads();
  // An expert's first row, end and first pair, read from the table once per
  // expert; a pair's rows are then scalar arithmetic (no LDS read and wait).
  struct ExpRows {
    int s, e, pb;
  };
  auto exp_rows = [&](int g) {
    ExpRows x;
    x.s = __builtin_amdgcn_readfirstlane(g_start[g]);
    x.e = __builtin_amdgcn_readfirstlane(g_start[g + 1]);
    x.pb = __builtin_amdgcn_readfirstlane(p_base[g]);
    return x;
  };
  auto rows_of = [&](const ExpRows& x, int p, int& r0, int& r1) {   // as pair_rows
    const int tile = x.s / kTileM + (p - x.pb);
    r0 = max(x.s, tile * kTileM);
    r1 = min(x.e, (tile + 1) * kTileM);
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave >> 1, wn = wave & 1;
  const int kt_n = K / BMK;
  // work item j of expert g = (n tile j / kt_n, k tile j % kt_n); it goes to
  // block (o_g + j) mod nb (see build_item_schedule), so a block walks the
  // experts in order and takes every nb-th item of each from its first one.
  // Items of one expert are spread over every block (and so over every XCD).
  auto first_j = [&](int g) {
    const int j = (int)blockIdx.x - (int)i_off[g];
    return __builtin_amdgcn_readfirstlane(j < 0 ? j + nb : j);
  };

  // ---- per-lane copy offsets within a chunk (item-independent part) and operand read offsets
  uint32_t va[kALoadsG], vb[kBLoadsG];
#pragma unroll
  for (int j = 0; j < kALoadsG; ++j) {
    const int row = (kALoadsG * wave + j) * C::kARows + lane / C::kAChunks;
    const int ch = (lane % C::kAChunks) ^ C::a_key(row);
    va[j] = (uint32_t)row * (uint32_t)K + (uint32_t)(ch * 16);
  }
#pragma unroll
  for (int j = 0; j < kBLoadsG; ++j) {
    const int row = (kBLoadsG * wave + j) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);
    vb[j] = (uint32_t)row * (uint32_t)N + (uint32_t)(ch * 16);
  }
  const int Lg = lane & 15;
  const int rbase = (lane >> 4) * 8 + (Lg >> 1);      // + 32 * s
  int a_rd[4], b_rd[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) a_rd[f] = C::l_slot(rbase, wk * 4 + f) + 8 * (Lg & 1);
#pragma unroll
  for (int j = 0; j < 4; ++j) b_rd[j] = kAStage + C::d_slot(rbase, wn * 4 + j) + 8 * (Lg & 1);
  // the rescale's scales in a stage slot: sL[wk*64 + f*16 + lane%16], sD[wn*64 + j*16 + 4*(lane/16) + 0..3]
  const int sl_rd = kAStage + kBStage + 4 * (wk * 64 + Lg);
  const int sd_rd = kAStage + kBStage + 4 * BMK + 4 * (wn * 64 + 4 * (lane >> 4));

  // ---- copy side: the next (item, pair, chunk) to copy, stages run ahead of the compute side
  int ig = 0, ij = first_j(0), ikt = 0, int_ = 0, ip = 0, ip1 = 0, ic = 0, inc = 0, irows = 0;
  ExpRows ix{0, 0, 0};
  auto set_pair = [&]() {   // chunks and padded rows of the copy side's pair ip
    int r0, r1;
    rows_of(ix, ip, r0, r1);
    irows = (r1 - r0 + kSub - 1) / kSub * kSub;
    inc = (irows + kChunk - 1) / kChunk;
  };
  auto seek = [&]() {   // first item at or after (ig, ij) whose expert has rows
    while (ig < G && (ij >= per_g || p_base[ig + 1] == p_base[ig])) {
      ++ig;
      if (ig < G) ij = first_j(ig);
    }
    if (ig < G) {
      ig = __builtin_amdgcn_readfirstlane(ig);
      ij = __builtin_amdgcn_readfirstlane(ij);
      ikt = ij % kt_n;
      int_ = ij / kt_n;
      ix = exp_rows(ig);
      ip = ix.pb;
      ip1 = __builtin_amdgcn_readfirstlane(p_base[ig + 1]);
      ic = 0;
      set_pair();
    }
  };
  int tI = 0;
  // copy parameters of the next chunk (ii, ip, ic)
  // the copy of a pair's last stage may run past its rows (padded with zero
  // codes to a multiple of 32): the buffer range ends there, so those loads
  // return zeros and the stage's MFMAs add nothing for them
  auto copy_rsrc_a = [&]() { return make_rsrc(ql + (size_t)ip * kTileM * K, (uint32_t)irows * (uint32_t)K); };
  auto copy_rsrc_b = [&]() { return make_rsrc(qd + (size_t)ip * kTileM * N, (uint32_t)irows * (uint32_t)N); };
  uint32_t va_i[kALoadsG], vb_i[kBLoadsG];      // copy offsets with the item's column origin
  auto set_item_offsets = [&]() {
#pragma unroll
    for (int j = 0; j < kALoadsG; ++j) va_i[j] = va[j] + (uint32_t)ikt * BMK;
#pragma unroll
    for (int j = 0; j < kBLoadsG; ++j) vb_i[j] = vb[j] + (uint32_t)int_ * BNN;
  };
  // this wave's slice of the pair's scales (see StageCopy)
  const bool s_is_l = wave < C::kSlicesL;
  const int s_part = s_is_l ? wave : (wave - C::kSlicesL) & 1;
  const uint32_t s_lds = (s_is_l ? 0u : 4u * BMK) + 256u * (uint32_t)s_part;
  // The slice's source is written without a select between the copy-side
  // tile indices (the optimizer turns such a select into one between their
  // addresses, which pins them in scratch): per-wave multipliers, opaque to it.
  const float* s_base = s_is_l ? sl : sd;
  const int s_stride = __builtin_amdgcn_readfirstlane(s_is_l ? K : N);
  const int s_mul_k = __builtin_amdgcn_readfirstlane(s_is_l ? BMK : 0);
  const int s_mul_n = __builtin_amdgcn_readfirstlane(s_is_l ? 0 : BNN);
  auto stage_copy = [&]() {
    StageCopy<C> cp;
    cp.ra = copy_rsrc_a();
    cp.rb = copy_rsrc_b();
    cp.rs = make_rsrc(s_base + (size_t)ip * s_stride, 4u * (uint32_t)s_stride);
#pragma unroll
    for (int j = 0; j < kALoadsG; ++j) cp.va[j] = va_i[j];
#pragma unroll
    for (int j = 0; j < kBLoadsG; ++j) cp.vb[j] = vb_i[j];
    cp.soa = (uint32_t)ic * kChunk * (uint32_t)K;
    cp.sob = (uint32_t)ic * kChunk * (uint32_t)N;
    cp.vs = 4u * (uint32_t)(ikt * s_mul_k + int_ * s_mul_n + 64 * s_part + lane);
    cp.s_lds = s_lds;
    return cp;
  };
  auto advance = [&]() {
    ++tI;
    if (++ic == inc) {
      ic = 0;
      if (++ip == ip1) {
        ij += nb;
        seek();
        set_item_offsets();
      } else {
        set_pair();
      }
    }
  };
  auto issue = [&]() {          // prologue copies (nothing is read yet)
    uint8_t* St = smem + (tI % kStagesG) * kStageG;
    const StageCopy<C> cp = stage_copy();
#pragma unroll
    for (int j = 0; j < kALoadsG; ++j) dma16(cp.ra, St + (kALoadsG * wave + j) * 1024, cp.va[j], cp.soa);
#pragma unroll
    for (int j = 0; j < kBLoadsG; ++j) dma16(cp.rb, St + kAStage + (kBLoadsG * wave + j) * 1024, cp.vb[j], cp.sob);
    dma4(cp.rs, St + kAStage + kBStage + cp.s_lds, cp.vs, 0);
    advance();
  };
  seek();
  set_item_offsets();
  for (int t = 0; t < kStagesG - 1 && ig < G; ++t) issue();

  // ---- compute side
  v4f tot[4][4], part[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tot[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
      part[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
  int tC = 0;
  for (int g = 0; g < G; ++g) {
  const ExpRows cx = exp_rows(g);
  const int p_end = __builtin_amdgcn_readfirstlane(p_base[g + 1]);
  for (int it = first_j(g); it < per_g; it += nb) {
    const int kt = it % kt_n, nt = it / kt_n;
    for (int p = cx.pb; p < p_end; ++p) {
      // the pair's rows padded to 32: its last chunk runs only the sub-steps they cover
      int pr0, pr1;
      rows_of(cx, p, pr0, pr1);
      const int rpad = (pr1 - pr0 + kSub - 1) / kSub * kSub;
      const int nc = (rpad + kChunk - 1) / kChunk;
      for (int c = 0; c < nc; ++c, ++tC) {
        // stage tC landed in every wave's copy (only the copies issued after
        // it may still be in flight; other loads and stores only make the
        // wait stricter); stage tC-1's buffer is free for the next copy
        const int pending = tI - 1 - tC;
        static_assert(kStagesG == 3 || kStagesG == 4, "one wait per possible count below");
        if (kStagesG == 4 && pending >= 2) wait_vmem_lds<(kStagesG == 4 ? 2 : 1) * kLoadsG>();
        else if (pending >= 1) wait_vmem_lds<kLoadsG>();
        else wait_vmem_lds<0>();
        barrier_only();
        const bool copy = ig < G;
        uint8_t* wr = smem + (tI % kStagesG) * kStageG;
        const uint8_t* rd = smem + (tC % kStagesG) * kStageG;
        const int nsub = min(kChunk, rpad - c * kChunk) / kSub;
        tgmm_stage<GRAD_E5M2, C>(wr, rd, copy, stage_copy(), wave, a_rd, b_rd, nsub, c == nc - 1, sl_rd,
                                             sd_rd, part, tot);
        if (copy) advance();
      }
    }
    // ---- store the tile (zeros for an expert without rows).
    // Lane (a = lane%16, b = lane/16) holds, for each f and j, row
    // k = wk*64 + f*16 + a and columns n = wn*64 + 16j + 4b .. +3, so lanes
    // a and a^8 hold the two 64-byte halves of the same cache lines (j even /
    // odd).  They swap one half (a DPP rotate by 8 within each row of 16
    // lanes, masked to the receiving lanes) so that each store writes 8 rows
    // x 128 contiguous bytes: streaming stores of half lines run at about
    // half the HBM write rate of whole lines.
    float* out = drhs + ((size_t)g * K + (size_t)kt * BMK) * N + (size_t)nt * BNN;
    const int a8 = lane & 7, hi8 = (lane >> 3) & 1;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      float* orow = out + (size_t)(wk * 64 + f * 16 + a8) * N + wn * 64 + 16 * hi8 + 4 * (lane >> 4);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const v4f lo = tot[f][2 * m], hi = tot[f][2 * m + 1];
        v4f r0, r1;   // rows a8 and a8 + 8 of the 16-row block, columns 32m + 16*hi8 + 4b
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // plain scalars: bit-casting a vector element directly reads element 0
          const int l = __builtin_bit_cast(int, (float)lo[r]), h = __builtin_bit_cast(int, (float)hi[r]);
          r0[r] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(l, h, 0x128, 0xf, 0xc, false));
          r1[r] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(h, l, 0x128, 0xf, 0x3, false));
        }
        __builtin_nontemporal_store(r0, reinterpret_cast<v4f*>(orow + 32 * m));
        __builtin_nontemporal_store(r1, reinterpret_cast<v4f*>(orow + (size_t)8 * N + 32 * m));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) tot[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    }
  }
  }
}

}  // namespace

size_t tgmm_workspace_bytes(long long M, long long K, long long N, int G) {
  const long long tmax = (M + kTileM - 1) / kTileM + G - 1;
  if (tmax <= 0) return 0;
  const size_t a = 256;
  auto al = [&](size_t x) { return (x + a - 1) / a * a; };
  return al((size_t)tmax * kTileM * K) + al((size_t)tmax * kTileM * N) + al((size_t)tmax * K * 4) +
         al((size_t)tmax * N * 4) + al((size_t)G * 4);
}

namespace {
size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// The GEMM's launch geometry: k-tile rows, ring-stage rows, items per expert, blocks.
struct GemmGeom {
  int bmk, chunk, per_g, nb;
};
GemmGeom gemm_geom(int G, int K, int N) {
  GemmGeom q;
  q.bmk = K % 256 == 0 ? 256 : 128;
  q.chunk = q.bmk == 256 ? TgCfg<256>::kChunk : TgCfg<128>::kChunk;
  const int per_cu = q.bmk == 256 ? TgCfg<256>::kBlocksPerCU : TgCfg<128>::kBlocksPerCU;
  q.per_g = (K / q.bmk) * (N / TgCfg<256>::BNN);
  // persistent: as many blocks as stay resident at once
  q.nb = (int)std::min<long long>((long long)G * q.per_g, (long long)per_cu * device_cu_count());
  return q;
}
// Whether the prep pass computes the item deal for this geometry (else the GEMM deals round-robin).
bool schedule_fits(int G, const GemmGeom& q) { return G <= kMaxSchedGroups && q.nb <= kMaxSchedBlocks && q.nb >= 1; }

template <int BMK>
hipError_t launch_tgmm_gemm_bmk(const uint8_t* ql, const uint8_t* qd, const float* sl, const float* sd,
                                const int* group_sizes, const int* sched, int G, int M, int K, int N, int nb,
                                bool grad_e5m2, float* drhs, hipStream_t stream) {
  using C = TgCfg<BMK>;
  const size_t lds = C::kLds + sizeof(int) * 2 * ((size_t)G + 1) + sizeof(uint16_t) * (size_t)G;
  const dim3 grid((unsigned)nb);
  if (grad_e5m2)
    hipLaunchKernelGGL((tgmm_gemm_kernel<true, BMK>), grid, dim3(C::kThreads), lds, stream, ql, qd, sl, sd,
                       group_sizes, sched, G, M, K, N, drhs);
  else
    hipLaunchKernelGGL((tgmm_gemm_kernel<false, BMK>), grid, dim3(C::kThreads), lds, stream, ql, qd, sl, sd,
                       group_sizes, sched, G, M, K, N, drhs);
  return hipGetLastError();
}

// sched: the item deal the prep pass wrote, or null for the round-robin deal.
hipError_t launch_tgmm_gemm(const uint8_t* ql, const uint8_t* qd, const float* sl, const float* sd,
                            const int* group_sizes, const int* sched, int G, int M, int K, int N, bool grad_e5m2,
                            float* drhs, hipStream_t stream) {
  const GemmGeom q = gemm_geom(G, K, N);
  if (q.bmk == 256)
    return launch_tgmm_gemm_bmk<256>(ql, qd, sl, sd, group_sizes, sched, G, M, K, N, q.nb, grad_e5m2, drhs, stream);
  return launch_tgmm_gemm_bmk<128>(ql, qd, sl, sd, group_sizes, sched, G, M, K, N, q.nb, grad_e5m2, drhs, stream);
}
}  // namespace

size_t tgmm_dense_workspace_bytes(long long M, long long K, long long N, int G) {
  const long long rc = (M + kDenseRows - 1) / kDenseRows;
  return tgmm_workspace_bytes(M, K, N, G) + al256((size_t)M * K) + al256((size_t)M * 4) + al256((size_t)M * N) +
         al256((size_t)rc * N * 4) + al256((size_t)N * 4);
}

hipError_t launch_tgmm_dense(const uint16_t* lhs, const uint16_t* dout, const int* group_sizes, int G, int M, int K,
                             int N, bool grad_e5m2, float* drhs, float* dbg_srow, float* dbg_scol, void* ws,
                             int* status, hipStream_t stream) {
  const long long tmax = (M + kTileM - 1) / kTileM + G - 1;
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* ql = base;
  uint8_t* qd = base + al256((size_t)tmax * kTileM * K);
  float* sl = reinterpret_cast<float*>(qd + al256((size_t)tmax * kTileM * N));
  float* sd = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(sl) + al256((size_t)tmax * K * 4));
  uint8_t* dense = base + tgmm_workspace_bytes(M, K, N, G);
  const int rc = (M + kDenseRows - 1) / kDenseRows;
  uint8_t* qLd = dense;
  float* srow = reinterpret_cast<float*>(qLd + al256((size_t)M * K));
  uint8_t* qDd = reinterpret_cast<uint8_t*>(srow) + al256((size_t)M * 4);
  float* partial = reinterpret_cast<float*>(qDd + al256((size_t)M * N));
  float* scol = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(partial) + al256((size_t)rc * N * 4));
  int* sched = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(sd) + al256((size_t)tmax * N * 4));
  const GemmGeom q = gemm_geom(G, K, N);
  const bool use_sched = M > 0 && tmax > 0 && schedule_fits(G, q);
  if (dbg_srow) srow = dbg_srow;
  if (dbg_scol) scol = dbg_scol;
  if (M > 0) {
    hipError_t e = launch_quant_rows_e4m3_all(lhs, M, K, qLd, srow, stream);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)rc, (unsigned)((N + kDenseCols - 1) / kDenseCols));
    hipLaunchKernelGGL(dense_colmax_kernel, grid, dim3(256), 0, stream, dout, srow, M, N, partial);
    hipLaunchKernelGGL(dense_colscale_kernel, dim3((unsigned)((N + 31) / 32)), dim3(256), 0, stream, partial, rc, N,
                       grad_e5m2 ? kE5M2Max : kE4M3Max, scol);
    if (grad_e5m2)
      hipLaunchKernelGGL(dense_quant_kernel<true>, grid, dim3(256), 0, stream, dout, srow, scol, M, N, qDd);
    else
      hipLaunchKernelGGL(dense_quant_kernel<false>, grid, dim3(256), 0, stream, dout, srow, scol, M, N, qDd);
    if (tmax > 0)
      hipLaunchKernelGGL(dense_gather_kernel, dim3((unsigned)tmax, (unsigned)(K / kPrepCols + N / kPrepCols)),
                         dim3(kThreads), 0, stream, qLd, qDd, scol, group_sizes, G, M, K, N, ql, qd, sl, sd, status,
                         use_sched ? sched : nullptr, q.chunk, q.per_g, q.nb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_tgmm_gemm(ql, qd, sl, sd, group_sizes, use_sched ? sched : nullptr, G, M, K, N, grad_e5m2, drhs,
                          stream);
}

hipError_t launch_tgmm_quant(const uint16_t* lhs, const uint16_t* dout, const int* group_sizes, int G, int M, int K,
                             int N, bool grad_e5m2, float* drhs, float* dbg_sl, float* dbg_sd, void* ws,
                             int* status, hipStream_t stream) {
  const long long tmax = (M + kTileM - 1) / kTileM + G - 1;
  const size_t a = 256;
  auto al = [&](size_t x) { return (x + a - 1) / a * a; };
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* ql = base;
  uint8_t* qd = base + al((size_t)tmax * kTileM * K);
  float* sl = reinterpret_cast<float*>(qd + al((size_t)tmax * kTileM * N));
  float* sd = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(sl) + al((size_t)tmax * K * 4));
  int* sched = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(sd) + al((size_t)tmax * N * 4));
  const GemmGeom q = gemm_geom(G, K, N);
  const bool use_sched = M > 0 && tmax > 0 && schedule_fits(G, q);
  if (dbg_sl) sl = dbg_sl;
  if (dbg_sd) sd = dbg_sd;
  if (tmax > 0 && M > 0) {
    dim3 grid((unsigned)(K / kPrepCols + N / kPrepCols), (unsigned)tmax);
    int* sp = use_sched ? sched : nullptr;
    if (grad_e5m2)
      hipLaunchKernelGGL(tgmm_prep_kernel<true>, grid, dim3(kThreads), 0, stream, lhs, dout, group_sizes, G, M, K,
                         N, ql, qd, sl, sd, status, sp, q.chunk, q.per_g, q.nb);
    else
      hipLaunchKernelGGL(tgmm_prep_kernel<false>, grid, dim3(kThreads), 0, stream, lhs, dout, group_sizes, G, M, K,
                         N, ql, qd, sl, sd, status, sp, q.chunk, q.per_g, q.nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_tgmm_gemm(ql, qd, sl, sd, group_sizes, use_sched ? sched : nullptr, G, M, K, N, grad_e5m2, drhs,
                          stream);
}

}  // namespace fp8gmm

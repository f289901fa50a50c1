// Native FP8 forward grouped matmul ("MoE: native FP8 QAT for routed-expert
// GMMs", Description and Data flow table: the wi/wo forward GMMs run FP8 x FP8
// with f32 accumulation, reading the e4m3 weight codes and the per-channel f32
// scale directly; Implementation: gmm_silu_fp8 fuses SwiGLU into wi).
//
// out[r, n] = bf16( (sum_k dec(aq[r,k]) * dec(codes[g,k,n])) * ascale[r] * wscale[g,n] )
// for every valid row r of expert g; with SwiGLU the columns are [gate | up]
// and out[r, i] = bf16( silu(y[r, i]) * y[r, I + i] ), I = N/2, and, when the
// caller asks for it, the pre-activation preact[r, n] = bf16(y[r, n]) (the
// values gmm_fp8_fwd would return) is kept for the fused dSwiGLU backward.
//
// Tiling (gfx950): a block owns a 256-row x BN-column output tile of one
// expert, BN = 256 (or 128 when N is not a multiple of 256; for SwiGLU 128
// gate + the matching 128 up columns).  Eight waves, two per SIMD, own
// 64 x BN/2 each (128 or 64 f32 accumulators per lane); the second wave on
// a SIMD issues MFMAs while the first waits on LDS or on its copies.  K
// advances 64 bytes per stage through a four-stage LDS ring:
//  * both tiles are copied HBM/L2 -> LDS by buffer loads with the LDS
//    destination, issued four stages ahead and spread over the MFMAs of a
//    stage (a stage's buffer is free once its operands are in registers);
//  * the activation tile is row-major, the weight tile keeps the natural
//    [k][n] layout; 16-byte chunks are XOR-swizzled so that the operand reads
//    hit distinct banks;
//  * the weight operand is read with the transposing ds_read_tr8_b64 (8
//    consecutive k of one column per lane), so the N-contiguous codes need no
//    transpose pass;
//  * one barrier per stage; after it each operand fragment of the next stage
//    is reread in place right after the last MFMA that uses the current one.
// The 32x32x64 MFMA takes the weight as its first operand, which makes each
// lane own one row and groups of four consecutive output columns: the
// epilogue scales, optionally applies SwiGLU, and stores 8-byte bf16 groups.
//
// Scheduling: every block rebuilds the expert table from group_sizes (a wave
// scan), maps its id to a (global m-tile, n-tile) pair in an m-grouped order
// (one m-tile of each group per XCD), and exits if it has no tile.  Tiles are aligned to each
// expert's first row; rows past an expert's end are never read (the load row
// is clamped inside the expert) and never written.
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace fp8gmm {
namespace {

constexpr int BM = 256;
constexpr int BK = 64;              // K bytes per stage
constexpr int kStages = 4;
constexpr int kThreads = 512;       // 8 waves, two per SIMD
constexpr int kGroupM = 8;

constexpr int kScaleBytes = 2048;   // the tile's 256 column scales, then its 256 row scales
template <int BN>
constexpr int stage_bytes() { return BM * BK + BK * BN; }
template <int BN>
constexpr int lds_main() { return kStages * stage_bytes<BN>() + kScaleBytes; }
static_assert(lds_main<256>() + sizeof(int) * (3 * kMaxGroups + 1) <= 160 * 1024,
              "ring + tile scales + expert table fit the LDS");

// 16-byte chunk swizzles: 16 lanes reading 16 consecutive activation rows at
// one chunk, and two transposing-read groups (8 weight rows each, adjacent
// chunks), hit distinct banks.
__device__ __forceinline__ int a_swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 2) & 3)) << 4); }
//   FP8 weights: a transposing-read group covers 8 weight rows x 16 bytes;
//   bf16 weights: 4 weight rows x 32 bytes (rows are 2*BN bytes).
template <bool BF16, int BN>
__device__ __forceinline__ int b_key(int k) {
  return BF16 ? ((k & 3) << 2) : (BN == 256 ? ((k & 7) << 1) : (((k >> 1) & 3) << 1));
}
template <bool BF16, int BN>
__device__ __forceinline__ int b_swz(int k, int chunk) {
  return k * (BF16 ? 2 * BN : BN) + ((chunk ^ b_key<BF16, BN>(k)) << 4);
}

// Transposing read of four consecutive k (rows) of one bf16 column: within each
// 16-lane group lane i receives element j from addr[4j + (i>>2)] + 2*(i&3)
// bytes, addr[L] being lane L's address.
__device__ __forceinline__ v2i lds_read_tr16(const void* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4s, const_cast<void*>(p)));
  return __builtin_bit_cast(v2i, v);
}

// BF16 = false: the FP8 forward (aq / codes are e4m3 bytes, scaled epilogue).
// BF16 = true: the bf16 measurement arm on the same schedule, ring and wave
// layout: aq / codes hold bf16 activations / weights, a stage still moves 64
// bytes of every activation row (32 k) and 32 weight rows of 2*BN bytes, each
// fragment takes two 32x32x16 bf16 MFMAs, and the epilogue has no scales.
// VAR (FP8, no SwiGLU, 128-column tiles): the ops-level LHS-quantization
// variants ("MoE: native FP8 QAT for routed-expert GMMs", Implementation:
// lhs_quant_block_size, rhs_scale_first; the bf16 accumulator of the earlier
// default).  Bit 1: one activation scale per 512 columns (ascale is
// [M, ceil(K/512)]); every 8 stages the block's accumulators are scaled and
// folded into a running total.  Bit 2: that total is a bf16 accumulator
// (rounded to bf16 after every fold).  Bit 4: the weight scale is applied
// before the activation scale.
template <bool BF16, bool SWIGLU, int BN, int VAR = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void gmm_fp8_fwd_kernel(const uint8_t* __restrict__ aq, const float* __restrict__ ascale,
                        const uint8_t* __restrict__ codes, const float* __restrict__ wscale,
                        const int* __restrict__ group_sizes, int G, int M, int K, int N,
                        uint16_t* __restrict__ out, uint16_t* __restrict__ preact, int* status) {
  constexpr int NJ = BN / 64;                       // 32-column fragments per wave (BN/2 columns)
  constexpr int MI = 2;                             // 32-row fragments per wave (64 rows)
  constexpr int kEl = BF16 ? 2 : 1;                 // bytes per element
  constexpr int kStageBytes = stage_bytes<BN>();
  constexpr int kBRow = BN * kEl;                   // bytes per weight-tile row
  constexpr int kBChunks = kBRow / 16;              // 16-byte chunks per weight-tile row
  constexpr int kALoads = BM * BK / 1024 / 8;       // 1 KB wave-wide copies per wave per stage
  constexpr int kBLoads = BK * BN / 1024 / 8;
  constexpr int kLoads = kALoads + kBLoads;
  constexpr int kBRowsPerLoad = 1024 / kBRow;
  static_assert(!SWIGLU || BN == 256, "SwiGLU pairs 2 gate with 2 up fragments per wave");
  static_assert(VAR == 0 || (!BF16 && !SWIGLU && BN == 128), "variants: FP8, plain epilogue, 128 columns");
  constexpr bool kBlockQ = (VAR & 1) != 0, kAccBf16 = (VAR & 2) != 0, kRhsFirst = (VAR & 4) != 0;
  static_assert(kLoads * (kStages - 1) < 64, "outstanding copies fit vmcnt");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* t_start = reinterpret_cast<int*>(smem + lds_main<BN>());
  int* t_end = t_start + G;
  int* t_pre = t_end + G;

  build_group_table(group_sizes, G, M, BM, GroupTable{t_start, t_end, t_pre}, status);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;          // 4 x 2 waves
  const int I = N >> 1;
  const int n_tiles = SWIGLU ? (I / (BN / 2)) : (N / BN);
  const int T = t_pre[G];
  const int total = T * n_tiles;
  const int b = blockIdx.x;
  if (b >= total) return;

  // ---- tile selection: groups of kGroupM m-tiles walk the n-tiles
  int mt, nt;
  raster_tile<kGroupM>(b, T, n_tiles, mt, nt);
  // values read from the LDS table are wave-uniform: keep them in scalar registers
  nt = __builtin_amdgcn_readfirstlane(nt);
  const int g = __builtin_amdgcn_readfirstlane(find_group(t_pre, G, mt));
  const int row0 = __builtin_amdgcn_readfirstlane(t_start[g] + (mt - t_pre[g]) * BM);
  const int rows = __builtin_amdgcn_readfirstlane(min(BM, t_end[g] - row0));

  // ---- buffer resources: the tile's activation rows and the expert's codes
  const BufRsrc ra = make_rsrc(aq + (size_t)row0 * K * kEl, (uint32_t)rows * (uint32_t)K * kEl);
  const BufRsrc rb = make_rsrc(codes + (size_t)g * K * N * kEl, (uint32_t)K * (uint32_t)N * kEl);
  uint32_t va[kALoads];                // activation chunk offsets (stage 0)
#pragma unroll
  for (int j = 0; j < kALoads; ++j) {
    const int r = (kALoads * wave + j) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    va[j] = (uint32_t)min(r, rows - 1) * (uint32_t)K * kEl + (uint32_t)(c << 4);
  }
  uint32_t vb[kBLoads];                // weight chunk offsets (stage 0)
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    constexpr int kHalf = kBChunks / 2, kChunkEl = 16 / kEl;
    const int kk = (kBLoads * wave + j) * kBRowsPerLoad + lane / kBChunks;
    const int c = (lane % kBChunks) ^ b_key<BF16, BN>(kk);
    int col;
    if (SWIGLU) col = (c < kHalf) ? nt * (BN / 2) + c * kChunkEl : I + nt * (BN / 2) + (c - kHalf) * kChunkEl;
    else col = nt * BN + c * kChunkEl;
    vb[j] = ((uint32_t)kk * (uint32_t)N + (uint32_t)col) * kEl;
  }

  // ---- per-lane LDS read offsets of the MFMA operands (within a stage)
  int a_rd[2];                         // + i * 32 rows
#pragma unroll
  for (int h = 0; h < 2; ++h) a_rd[h] = a_swz(wm * 64 + (lane & 31), 2 * (lane >> 5) + h);
  // Weight operand: lanes 0-31 take k 0..BK/2-1 of the stage (in bytes), lanes
  // 32-63 the rest; the activation operand uses the same split, so every MFMA
  // pairs the same k on both sides.
  int b_rd[NJ];                        // + t * (8 FP8 | 4 bf16) rows
  {
    const int gq = lane >> 4, Lg = lane & 15;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int tc;                          // first tile column of fragment j
      if (SWIGLU) tc = (j < 2) ? wn * 64 + 32 * j : 128 + wn * 64 + 32 * (j - 2);
      else tc = wn * (BN / 2) + 32 * j;
      if (BF16) {
        const int kk = (gq >> 1) * 16 + (Lg >> 2);
        b_rd[j] = BM * BK + b_swz<BF16, BN>(kk, (tc >> 3) + 2 * (gq & 1) + ((Lg & 3) >> 1)) + 8 * (Lg & 1);
      } else {
        const int kk = (gq >> 1) * 32 + (Lg >> 1);
        b_rd[j] = BM * BK + b_swz<BF16, BN>(kk, (tc >> 4) + (gq & 1)) + 8 * (Lg & 1);
      }
    }
  }

  auto issue_one = [&](uint8_t* S, int ks, int q) {   // copy number q (0 .. kLoads-1) of stage ks into S
    if (q < kALoads) dma16(ra, S + (kALoads * wave + q) * 1024, va[q], (uint32_t)ks * BK);
    else dma16(rb, S + BM * BK + (kBLoads * wave + q - kALoads) * 1024, vb[q - kALoads], (uint32_t)ks * BK * (uint32_t)N);
  };
  auto read_a = [&](const uint8_t* St, int i) {
    const uint8_t* S = St + i * 32 * BK;
    const v4i lo = *reinterpret_cast<const v4i*>(S + a_rd[0]);
    const v4i hi = *reinterpret_cast<const v4i*>(S + a_rd[1]);
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto read_b = [&](const uint8_t* St, int j) {
    const uint8_t* S = St + b_rd[j];
    v8i r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v2i v = BF16 ? lds_read_tr16(S + t * 4 * kBRow) : lds_read_tr8(S + t * 8 * kBRow);
      r[2 * t] = v[0];
      r[2 * t + 1] = v[1];
    }
    return r;
  };
  // one stage of fragment (i, j): FP8 one 32x32x64, bf16 two 32x32x16 (the
  // halves of the lane's 32 bytes)
  auto mma = [&](const v8i& bw, const v8i& av, const v16f& c) {
    if (BF16) {
      const v16f c1 = mfma_bf16_32x32x16(__builtin_bit_cast(v8bf, (v4i){bw[0], bw[1], bw[2], bw[3]}),
                                         __builtin_bit_cast(v8bf, (v4i){av[0], av[1], av[2], av[3]}), c);
      return mfma_bf16_32x32x16(__builtin_bit_cast(v8bf, (v4i){bw[4], bw[5], bw[6], bw[7]}),
                                __builtin_bit_cast(v8bf, (v4i){av[4], av[5], av[6], av[7]}), c1);
    }
    return mfma_e4m3_32x32x64(bw, av, c);
  };

  v16f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K * kEl / BK;

  // ---- variants: fold stage-block b's accumulators into the running total
  v16f tot[MI][NJ];
  if (kBlockQ) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) tot[i][j][r] = 0.f;
  }
  auto fold = [&](int blk) __attribute__((always_inline)) {
    const int nb = (K + 511) >> 9;
    const float* wsg = wscale + (size_t)g * N;
    const int hl = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int ml = wm * 64 + i * 32 + (lane & 31);
      const float sb = ml < rows ? ascale[(size_t)(row0 + ml) * nb + blk] : 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4f sc = *reinterpret_cast<const v4f*>(wsg + nt * BN + wn * (BN / 2) + 32 * j + 8 * q + hl);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = acc[i][j][4 * q + e];
            const float t = kRhsFirst ? (a * sc[e]) * sb : (a * sb) * sc[e];
            const float v = tot[i][j][4 * q + e] + t;
            tot[i][j][4 * q + e] = kAccBf16 ? __builtin_bit_cast(float, pack_bf16x2(v, 0.f) << 16) : v;
            acc[i][j][4 * q + e] = 0.f;
          }
        }
    }
  };
  auto maybe_fold = [&](int k) __attribute__((always_inline)) {
    if (kBlockQ && ((k & 7) == 7 || k + 1 == nk)) fold(k >> 3);
  };

  // ---- the tile's scales go to LDS ahead of stage 0 (they are older than
  // stage 0's copies, so they have landed whenever it has): wave 0 copies the
  // 256 column scales (SwiGLU: the 128 gate, then the 128 up columns), wave 1
  // the 256 row scales (rows past the tile's end read as zero).  The epilogue
  // then reads no global memory.
  constexpr bool kLdsScales = !BF16 && VAR == 0;
  uint8_t* const sc_lds = smem + kStages * kStageBytes;
  if (kLdsScales && wave == 0) {
    const int l = (BN == 256) ? lane : (lane & 31);
    int col;
    if (SWIGLU) col = (l < 32) ? nt * (BN / 2) + 4 * l : I + nt * (BN / 2) + 4 * (l - 32);
    else col = nt * BN + 4 * l;
    dma16(make_rsrc(wscale + (size_t)g * N, (uint32_t)N * 4u), sc_lds, (uint32_t)col * 4u, 0);
  } else if (kLdsScales && wave == 1) {
    // one dword per lane and copy, so each row is range-checked on its own
    const BufRsrc rr = make_rsrc(ascale + row0, (uint32_t)rows * 4u);
#pragma unroll
    for (int t = 0; t < 4; ++t) dma4(rr, sc_lds + 1024 + 256 * t, (uint32_t)lane * 4u, (uint32_t)t * 256u);
  }

  // ---- prologue: stages 0..3 in flight, stage 0 landed and in registers
  const int pre = min(nk, kStages);
  for (int s = 0; s < pre; ++s)
#pragma unroll
    for (int q = 0; q < kLoads; ++q) issue_one(smem + s * kStageBytes, s, q);
  if (pre >= 4) wait_vmem_lds<3 * kLoads>();
  else if (pre == 3) wait_vmem_lds<2 * kLoads>();
  else if (pre == 2) wait_vmem_lds<kLoads>();
  else wait_vmem_lds<0>();
  barrier_only();
  // A wave whose 64 rows all lie past the tile's last valid row (an expert's
  // short last tile) skips its operand reads and MFMAs; it still issues its
  // share of the copies and joins every barrier.  The two waves of a SIMD own
  // rows 0-127 and 128-255 of the tile, so a tile of at most 128 valid rows
  // keeps one wave's MFMAs per SIMD.
  const bool active = wm * 64 < rows;
  v8i a[MI], bf[NJ];
  if (active) {
#pragma unroll
    for (int i = 0; i < MI; ++i) a[i] = read_a(smem, i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bf[j] = read_b(smem, j);
  }

  // One stage.  ISSUE: copy stage ks+4 into this stage's buffer `wr` (its
  // operands are in registers; the barrier makes sure every wave's are);
  // MORE: stage ks+1 (buffer `rd`) exists and is reread into the registers as
  // they free up; WAITN: copies issued after stage ks+1 that may still be in
  // flight at the barrier; ACT: the wave computes (see above).  `wr` and `rd`
  // are distinct ring slots: marking them __restrict__ tells the compiler the
  // reads cannot depend on the copies issued here, so it adds no wait for them
  // (the wait + barrier above order the ring).
  auto step = [&](int ks, auto issue_c, auto more_c, auto waitn_c, auto act_c, uint8_t* __restrict__ wr,
                  const uint8_t* __restrict__ rd) {
    constexpr bool ISSUE = decltype(issue_c)::value;
    constexpr bool MORE = decltype(more_c)::value;
    constexpr int WAITN = decltype(waitn_c)::value;
    constexpr bool ACT = decltype(act_c)::value;
    v8i an[MI];
    if (MORE) {
      wait_vmem_lds<WAITN * kLoads>();
      barrier_only();
      if constexpr (ACT) {
#pragma unroll
        for (int i = 0; i < MI; ++i) an[i] = read_a(rd, i);
      }
      sched_fence();
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      prio_by_progress(j);
      if (ISSUE) {
#pragma unroll
        for (int q = j * kLoads / NJ; q < (j + 1) * kLoads / NJ; ++q) issue_one(wr, ks + kStages, q);
      }
      if constexpr (ACT) {
#pragma unroll
        for (int i = 0; i < MI; ++i) acc[i][j] = mma(bf[j], a[i], acc[i][j]);
        if (MORE) bf[j] = read_b(rd, j);
      }
      sched_fence();   // keep each refill between the MFMAs that surround it
    }
    if (MORE && ACT) {
#pragma unroll
      for (int i = 0; i < MI; ++i) a[i] = an[i];
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using W0 = std::integral_constant<int, 0>;
  using W1 = std::integral_constant<int, 1>;
  using W2 = std::integral_constant<int, 2>;
  auto slot = [&](int s) { return smem + (s % kStages) * kStageBytes; };
  auto run = [&](auto act_c) {
    constexpr bool ACT = decltype(act_c)::value;
    auto fold_if = [&](int k) __attribute__((always_inline)) {
      if constexpr (ACT) maybe_fold(k);
    };
    int ks = 0;
    for (; ks + kStages < nk; ++ks) {
      step(ks, T_{}, T_{}, W2{}, act_c, slot(ks), slot(ks + 1));
      fold_if(ks);
    }
    if (ks + 3 < nk) { step(ks, F_{}, T_{}, W2{}, act_c, slot(ks), slot(ks + 1)); fold_if(ks); ++ks; }
    if (ks + 2 < nk) { step(ks, F_{}, T_{}, W1{}, act_c, slot(ks), slot(ks + 1)); fold_if(ks); ++ks; }
    if (ks + 1 < nk) { step(ks, F_{}, T_{}, W0{}, act_c, slot(ks), slot(ks + 1)); fold_if(ks); ++ks; }
    step(ks, F_{}, F_{}, W0{}, act_c, slot(ks), slot(ks));
    fold_if(ks);
  };
  if (active) run(T_{});
  else run(F_{});
  prio_by_progress<3>();

  // ---- epilogue: lane owns row wm*64 + i*32 + lane%32 and, per fragment j,
  // columns tc(j) + 8*q + 4*(lane/32) + 0..3 for q = 0..3
  const float* ws = BF16 ? nullptr : wscale + (size_t)g * N;
  const v4f ones = {1.f, 1.f, 1.f, 1.f};
  const int hl = 4 * (lane >> 5);
  // Lanes l and l+32 hold the same row: pq[q] holds columns 8q+0..3 (lane l)
  // or 8q+4..7 (lane l+32) of a 32-column fragment.  Trading two 8-byte groups
  // gives lane l columns 0-7 and 16-23 and lane l+32 columns 8-15 and 24-31, so
  // every store is 16 bytes and each store instruction writes 32 contiguous
  // bytes of every row it touches (with 8-byte stores the epilogue cost a
  // fifth of the short-K forward's time).
  auto store_frag = [&](uint16_t* rowp, const v2i* pq) __attribute__((always_inline)) {
    const bool lo = (lane & 32) == 0;
    const v2i s0 = lo ? pq[1] : pq[0], s1 = lo ? pq[3] : pq[2];
    const int r00 = __shfl_xor(s0[0], 32), r01 = __shfl_xor(s0[1], 32);
    const int r10 = __shfl_xor(s1[0], 32), r11 = __shfl_xor(s1[1], 32);
    const v4i x0 = lo ? (v4i){pq[0][0], pq[0][1], r00, r01} : (v4i){r00, r01, pq[1][0], pq[1][1]};
    const v4i x1 = lo ? (v4i){pq[2][0], pq[2][1], r10, r11} : (v4i){r10, r11, pq[3][0], pq[3][1]};
    *reinterpret_cast<v4i*>(rowp + (lo ? 0 : 8)) = x0;
    *reinterpret_cast<v4i*>(rowp + (lo ? 16 : 24)) = x1;
  };
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int ml = wm * 64 + i * 32 + (lane & 31);
    if (ml < rows) {
      const int row = row0 + ml;
      const float sr = (BF16 || kBlockQ) ? 1.f
                       : (kLdsScales ? reinterpret_cast<const float*>(sc_lds + 1024)[ml] : ascale[row]);
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          v2i pgq[4], puq[4];   // pre-activation of columns 8q + hl + 0..3, gate and up
          v2i poq[4];           // output of the same columns
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = nt * (BN / 2) + wn * 64 + 32 * j + 8 * q + hl;
            const v4f sg = BF16 ? ones : *reinterpret_cast<const v4f*>(sc_lds + 4 * (c - nt * (BN / 2)));
            const v4f su = BF16 ? ones : *reinterpret_cast<const v4f*>(sc_lds + 512 + 4 * (c - nt * (BN / 2)));
            float o[4], yg[4], yu[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              yg[e] = (acc[i][j][4 * q + e] * sr) * sg[e];
              yu[e] = (acc[i][j + 2][4 * q + e] * sr) * su[e];
              // silu through the hardware reciprocal (about 1 ulp) rather than an
              // IEEE division: the product is rounded to bf16 right after
              o[e] = yg[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-yg[e])) * yu[e];
            }
            poq[q][0] = (int)pack_bf16x2(o[0], o[1]);
            poq[q][1] = (int)pack_bf16x2(o[2], o[3]);
            pgq[q][0] = (int)pack_bf16x2(yg[0], yg[1]);
            pgq[q][1] = (int)pack_bf16x2(yg[2], yg[3]);
            puq[q][0] = (int)pack_bf16x2(yu[0], yu[1]);
            puq[q][1] = (int)pack_bf16x2(yu[2], yu[3]);
          }
          store_frag(out + (size_t)row * I + nt * (BN / 2) + wn * 64 + 32 * j, poq);
          if (preact) {
            // Lanes l and l+32 hold the same row, columns 8q+0..3 and 8q+4..7.  Trading one
            // 8-byte half per column pair makes each lane own 8 consecutive columns, so the
            // pre-activation leaves in 16-byte stores (with 8-byte stores the L2 writes
            // these lines back about twice).
            const bool lo = (lane & 32) == 0;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const v2i sg = lo ? pgq[2 * p + 1] : pgq[2 * p];
              const v2i su = lo ? puq[2 * p + 1] : puq[2 * p];
              const int rg0 = __shfl_xor(sg[0], 32), rg1 = __shfl_xor(sg[1], 32);
              const int ru0 = __shfl_xor(su[0], 32), ru1 = __shfl_xor(su[1], 32);
              const v4i g4 = lo ? (v4i){pgq[2 * p][0], pgq[2 * p][1], rg0, rg1}
                                : (v4i){rg0, rg1, pgq[2 * p + 1][0], pgq[2 * p + 1][1]};
              const v4i u4 = lo ? (v4i){puq[2 * p][0], puq[2 * p][1], ru0, ru1}
                                : (v4i){ru0, ru1, puq[2 * p + 1][0], puq[2 * p + 1][1]};
              const int cb = nt * (BN / 2) + wn * 64 + 32 * j + 16 * p + (lo ? 0 : 8);
              *reinterpret_cast<v4i*>(preact + (size_t)row * N + cb) = g4;
              *reinterpret_cast<v4i*>(preact + (size_t)row * N + I + cb) = u4;
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          v2i pq[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = nt * BN + wn * (BN / 2) + 32 * j + 8 * q + hl;
            const v4f sc = BF16 ? ones
                           : (kLdsScales ? *reinterpret_cast<const v4f*>(sc_lds + 4 * (c - nt * BN))
                                         : *reinterpret_cast<const v4f*>(ws + c));
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = kBlockQ ? tot[i][j][4 * q + e]
                             : (kRhsFirst ? (acc[i][j][4 * q + e] * sc[e]) * sr : (acc[i][j][4 * q + e] * sr) * sc[e]);
            pq[q][0] = (int)pack_bf16x2(v[0], v[1]);
            pq[q][1] = (int)pack_bf16x2(v[2], v[3]);
          }
          store_frag(out + (size_t)row * N + nt * BN + wn * (BN / 2) + 32 * j, pq);
        }
      }
    }
  }
}

}  // namespace

namespace {

template <bool BF16>
hipError_t launch_fwd_impl(const uint8_t* a, const float* ascale, const uint8_t* w, const float* wscale,
                           const int* group_sizes, int G, int M, int K, int N, bool swiglu, uint16_t* out,
                           uint16_t* preact, int* status, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const long long max_m_tiles = (M + BM - 1) / BM + G;
  const size_t table = sizeof(int) * (3 * (size_t)G + 1);
  if (swiglu) {
    const long long grid = max_m_tiles * ((N / 2) / 128);
    hipLaunchKernelGGL((gmm_fp8_fwd_kernel<BF16, true, 256>), dim3((unsigned)grid), dim3(kThreads),
                       (lds_main<256>() + table), stream, a, ascale, w, wscale, group_sizes, G, M, K, N, out, preact,
                       status);
  } else if (N % 256 == 0) {
    const long long grid = max_m_tiles * (N / 256);
    hipLaunchKernelGGL((gmm_fp8_fwd_kernel<BF16, false, 256>), dim3((unsigned)grid), dim3(kThreads),
                       (lds_main<256>() + table), stream, a, ascale, w, wscale, group_sizes, G, M, K, N, out, nullptr,
                       status);
  } else {
    const long long grid = max_m_tiles * (N / 128);
    hipLaunchKernelGGL((gmm_fp8_fwd_kernel<BF16, false, 128>), dim3((unsigned)grid), dim3(kThreads),
                       (lds_main<128>() + table), stream, a, ascale, w, wscale, group_sizes, G, M, K, N, out, nullptr,
                       status);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gmm_fp8_fwd(const uint8_t* aq, const float* ascale, const uint8_t* codes, const float* wscale,
                              const int* group_sizes, int G, int M, int K, int N, bool swiglu, uint16_t* out,
                              uint16_t* preact, int* status, hipStream_t stream) {
  return launch_fwd_impl<false>(aq, ascale, codes, wscale, group_sizes, G, M, K, N, swiglu, out,
                                swiglu ? preact : nullptr, status, stream);
}

hipError_t launch_gmm_fp8_fwd_variant(const uint8_t* aq, const float* ascale, const uint8_t* codes,
                                      const float* wscale, const int* group_sizes, int G, int M, int K, int N,
                                      bool block512, bool acc_bf16, bool rhs_first, uint16_t* out, int* status,
                                      hipStream_t stream) {
  const int var = (block512 ? 1 : 0) | (block512 && acc_bf16 ? 2 : 0) | (rhs_first ? 4 : 0);
  if (var == 0)
    return launch_fwd_impl<false>(aq, ascale, codes, wscale, group_sizes, G, M, K, N, false, out, nullptr, status,
                                  stream);
  if (M == 0) return hipSuccess;
  const long long grid = ((M + BM - 1) / BM + G) * (N / 128);
  const size_t lds = lds_main<128>() + sizeof(int) * (3 * (size_t)G + 1);
#define VLAUNCH(V)                                                                                         \
  hipLaunchKernelGGL((gmm_fp8_fwd_kernel<false, false, 128, V>), dim3((unsigned)grid), dim3(kThreads), lds,  \
                     stream, aq, ascale, codes, wscale, group_sizes, G, M, K, N, out, nullptr, status)
  switch (var) {
    case 1: VLAUNCH(1); break;
    case 3: VLAUNCH(3); break;
    case 4: VLAUNCH(4); break;
    case 5: VLAUNCH(5); break;
    default: VLAUNCH(7); break;
  }
#undef VLAUNCH
  return hipGetLastError();
}

hipError_t launch_gmm_bf16_fwd(const uint16_t* lhs, const uint16_t* w, const int* group_sizes, int G, int M, int K,
                               int N, bool swiglu, uint16_t* out, int* status, hipStream_t stream) {
  return launch_fwd_impl<true>(reinterpret_cast<const uint8_t*>(lhs), nullptr, reinterpret_cast<const uint8_t*>(w),
                               nullptr, group_sizes, G, M, K, N, swiglu, out, nullptr, status, stream);
}

}  // namespace fp8gmm

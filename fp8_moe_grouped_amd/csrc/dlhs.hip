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
// epilogue: every weight element is decoded exactly, multiplied by its f32
// scale and rounded to bf16 (the arithmetic of dequantize_fp8_codes) before
// it enters a bf16 MFMA with f32 accumulation.
//
// Tiling (gfx950): a block owns BM rows x BN output columns of one expert
// (BM = 256, or 64 when the buffer holds at most 64 rows per expert on
// average, where most rows of a 256-row tile would be padding; BN = 256, or
// 128 when K is not a multiple of 256).  Eight waves, two per SIMD, in a
// 2 x 4 grid own BM/2 rows x BN/4 columns each (up to 128 f32 accumulators
// per lane); the second wave on a SIMD issues MFMAs while the first waits or
// converts.  The contraction advances 64 per stage through a
// three-stage LDS ring (bf16 weights always use BN = 128 to fit), each holding
//   * the dout tile, [BM rows][64 bf16], 16-byte chunks XOR-swizzled;
//   * the weight tile in its natural [k][n] layout (n contiguous, which is the
//     contraction), [BN rows][64 codes] or [BN rows][64 bf16], swizzled;
//   * the 64 scales of the stage (every wave copies all of them, the same
//     bytes to the same place, so the copy needs no per-lane branch).
// Every byte reaches LDS through buffer loads with an LDS destination, issued
// at the top of a stage for two stages ahead; one barrier per stage, before
// the next stage is first read (on the 256-row code path one fragment before
// the stage's last, so that the next stage's codes can be read two fragments
// ahead).
//
// Inner loop: a wave keeps its BM/2-row dout operand of the stage in registers
// and streams its weight fragments (16 output columns each): the next
// fragment is read from LDS, decoded, scaled and rounded on the VALU between
// the 16 MFMAs of the current one (on the 256-row code path one output word,
// two weights, after every second MFMA, with scheduling fences between the
// pieces; the stage's scales are read once, one per
// lane, and a DPP row broadcast inside each multiply hands every lane the
// scale of its contraction index); during the
// last fragment the dout operand of the next stage is reread in place right
// after the MFMAs that last use each register.  Each lane reads 16 consecutive
// contraction values of a row, which the two 16x16x32 MFMAs of a stage take
// as their two 8-value halves; dout and the weight use the same assignment,
// so the order of summation is the same whether the weights arrive as codes
// or as bf16 (the bf16 path is the measurement arm and, fed with
// dequantize_fp8_codes' output, must reproduce the FP8-code result bit for
// bit).  The MFMA takes the weight as its first operand so each lane owns
// four consecutive output columns of one row.  Group scheduling and the
// never-read / never-written stale rows are as in the forward.
//
// dSwiGLU arm (the backward of the wo op gmm_dswiglu_fp8, "MoE: native FP8
// QAT for routed-expert GMMs", Implementation: _run_wo_gmm_dswiglu): the
// dLHS of wo is the gradient dh of h = silu(gate) * up, and the epilogue turns
// it into the gradient of the wi pre-activation [gate | up] (bf16 [M, 2K], as
// the wi forward kept it) without rounding dh:
//   d_gate = dh * up * silu'(gate),  d_up = dh * silu(gate),
//   silu'(z) = sigma(z) * (1 + z * (1 - sigma(z))),  sigma(z) = 1 / (1 + e^-z).
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace fp8gmm {
namespace {

constexpr int BKN = 64;                 // contraction (n) per stage
constexpr int kARow = BKN * 2;          // 128 bytes per dout tile row
constexpr int kThreads = 512;           // 8 waves, two per SIMD
constexpr int kGroupM = 8;

// BM: rows per block tile, 256, or 64 for skinny groups (a buffer with at
// most 64 rows per expert on average), where a 256-row tile would spend
// most of its MFMAs on padding rows.
template <bool FROM_CODES, int BN, int BM>
struct Cfg {
  static constexpr int NJ = BN / 64;                         // 16-column fragments per wave
  static constexpr int FBK = BM / 32;                        // 16-row fragments per wave (BM/2 rows)
  static constexpr int kWRow = FROM_CODES ? BKN : BKN * 2;   // bytes per weight tile row
  static constexpr int kABytes = BM * kARow;
  static constexpr int kWBytes = BN * kWRow;
  static constexpr int kSBytes = FROM_CODES ? 256 : 0;       // the stage's 64 scales
  static constexpr int kStage = kABytes + kWBytes + kSBytes;
  static constexpr int kStages = 3;
  static constexpr int kLds = kStages * kStage;
  static constexpr int kALoads = kABytes / 1024 / 8;          // 1 KB wave-wide copies per wave per stage
  static constexpr int kWLoads = kWBytes / 1024 / 8;
  static constexpr int kLoads = kALoads + kWLoads + (FROM_CODES ? 1 : 0);
  static_assert(kLoads < 64, "outstanding copies fit vmcnt");
  static_assert(kLds + sizeof(int) * (3 * kMaxGroups + 1) <= 160 * 1024, "ring + expert table fit the LDS");
};

// 16-byte chunk swizzles of the operand tiles.  An operand read has 16 lanes
// on 16 consecutive rows at one logical chunk (the four 16-lane rows of a
// wave at four chunks).  The XOR keys were chosen by measurement on gfx950
// (LDS bank-conflict cycles per ds_read_b128 over every linear key of the
// row's low four bits): these take 4 LDS cycles per read; the plain
// (row >> 1) / (row >> 2) keys took 8.
//   128-byte rows (dout, bf16 weights): chunk ^= row bit 1 | row bit 3 << 2
//   64-byte rows (weight codes):        chunk ^= row bit 3 << 1
__device__ __forceinline__ int a_key(int row) { return ((row >> 1) & 1) | (((row >> 3) & 1) << 2); }
__device__ __forceinline__ int w_key(int row) { return ((row >> 3) & 1) << 1; }
__device__ __forceinline__ int a_swz(int row, int chunk) { return row * 128 + ((chunk ^ a_key(row)) << 4); }
__device__ __forceinline__ int w_swz(int row, int chunk) { return row * 64 + ((chunk ^ w_key(row)) << 4); }

__device__ __forceinline__ v8bf as_bf(const v4i& v) { return __builtin_bit_cast(v8bf, v); }

// The value that lane I of this lane's 16-lane row holds (DPP row_newbcast;
// the compiler folds it into the multiply that consumes it).
template <int I>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + I, 0xf, 0xf, false));
}

// 8 codes (two dwords) -> 8 bf16 weights.  Lane i of a 16-lane row holds the
// scale of contraction index i of the row's 16; the codes are indices
// 8H .. 8H+7.
template <int H>
__device__ __forceinline__ v4i deq8(uint32_t w0, uint32_t w1, float srow) {
  const v2f a = dec_e4m3x2<false>(w0), b = dec_e4m3x2<true>(w0);
  const v2f c = dec_e4m3x2<false>(w1), d = dec_e4m3x2<true>(w1);
  return (v4i){(int)pack_bf16x2(a[0] * row_bcast<8 * H + 0>(srow), a[1] * row_bcast<8 * H + 1>(srow)),
               (int)pack_bf16x2(b[0] * row_bcast<8 * H + 2>(srow), b[1] * row_bcast<8 * H + 3>(srow)),
               (int)pack_bf16x2(c[0] * row_bcast<8 * H + 4>(srow), c[1] * row_bcast<8 * H + 5>(srow)),
               (int)pack_bf16x2(d[0] * row_bcast<8 * H + 6>(srow), d[1] * row_bcast<8 * H + 7>(srow))};
}

// Output word O (0..7) of a 16-code fragment: the two weights of
// contraction indices 2O, 2O+1 (deq8<O / 4>'s word O % 4, on its own).
template <int O>
__device__ __forceinline__ int deq_word(const v8i& r, float srow) {
  constexpr int H = O / 4, m = O % 4;
  const v2f v = dec_e4m3x2<(m & 1) != 0>((uint32_t)r[2 * H + (m >> 1)]);
  return (int)pack_bf16x2(v[0] * row_bcast<8 * H + 2 * m>(srow), v[1] * row_bcast<8 * H + 2 * m + 1>(srow));
}

__device__ __forceinline__ float bf16_lo(int v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
__device__ __forceinline__ float bf16_hi(int v) { return __builtin_bit_cast(float, (uint32_t)v & 0xffff0000u); }

// gradients of silu(g) * u from the gradient dh of the product (f32)
__device__ __forceinline__ void dswiglu1(float dh, float g, float u, float& dg, float& du) {
  const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  const float t = fmaf(g, 1.0f - sig, 1.0f);
  dg = dh * u * (sig * t);
  du = dh * (g * sig);
}

template <bool FROM_CODES, int BN, bool DSWIGLU, int BM>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void gmm_dlhs_kernel(const uint16_t* __restrict__ dout, const uint8_t* __restrict__ codes,
                     const float* __restrict__ wscale, const uint16_t* __restrict__ wbf16,
                     const int* __restrict__ group_sizes, int G, int M, int K, int N,
                     const uint16_t* __restrict__ preact, uint16_t* __restrict__ dlhs, int* status) {
  static_assert(!DSWIGLU || FROM_CODES, "the dSwiGLU epilogue belongs to the FP8-code path");
  using C = Cfg<FROM_CODES, BN, BM>;
  constexpr int NJ = C::NJ;
  constexpr int FBK = C::FBK;
  constexpr int S = C::kStages;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int* t_start = reinterpret_cast<int*>(smem + C::kLds);
  int* t_end = t_start + G;
  int* t_pre = t_end + G;

  build_group_table(group_sizes, G, M, BM, GroupTable{t_start, t_end, t_pre}, status);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;          // 2 x 4 waves
  const int n_tiles = K / BN;
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

  // ---- buffer resources and per-lane copy offsets (stage 0)
  const BufRsrc ra = make_rsrc(dout + (size_t)row0 * N, (uint32_t)rows * (uint32_t)N * 2u);
  const BufRsrc rw = FROM_CODES ? make_rsrc(codes + (size_t)g * K * N, (uint32_t)K * (uint32_t)N)
                                : make_rsrc(wbf16 + (size_t)g * K * N, (uint32_t)K * (uint32_t)N * 2u);
  const BufRsrc rs = make_rsrc(FROM_CODES ? wscale + (size_t)g * N : wscale, FROM_CODES ? (uint32_t)N * 4u : 0u);
  uint32_t va[C::kALoads];
#pragma unroll
  for (int j = 0; j < C::kALoads; ++j) {
    const int r = (C::kALoads * wave + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ a_key(r);
    va[j] = (uint32_t)min(r, rows - 1) * (uint32_t)N * 2u + (uint32_t)(c << 4);
  }
  uint32_t vw[C::kWLoads];
#pragma unroll
  for (int j = 0; j < C::kWLoads; ++j) {
    if (FROM_CODES) {
      const int kr = (C::kWLoads * wave + j) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ w_key(kr);
      vw[j] = (uint32_t)(nt * BN + kr) * (uint32_t)N + (uint32_t)(c << 4);
    } else {
      const int kr = (C::kWLoads * wave + j) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ a_key(kr);
      vw[j] = (uint32_t)(nt * BN + kr) * (uint32_t)N * 2u + (uint32_t)(c << 4);
    }
  }

  // ---- per-lane LDS read offsets (within a stage)
  const int q = lane >> 4;
  int a_rd[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) a_rd[s] = a_swz(wm * (BM / 2) + (lane & 15), 2 * q + s);   // + f * 2048
  int w_rd[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    w_rd[s] = C::kABytes + (FROM_CODES ? w_swz(wn * (16 * NJ) + (lane & 15), q)           // + j * 1024
                                       : a_swz(wn * (16 * NJ) + (lane & 15), 2 * q + s));  // + j * 2048
  // Lane l reads scale l of the stage: the 16 lanes of row q then hold the
  // scales of contraction indices 16q .. 16q+15, the ones the row's weight
  // values need (one conflict-free read per stage instead of each lane
  // reading the row's 16 scales from the same addresses).
  const int s_rd = C::kABytes + C::kWBytes + 4 * lane;

  // copy number c (0 .. kLoads-1) of stage ks into slot St
  auto issue_one = [&](uint8_t* St, int ks, int c) {
    if (c < C::kALoads) {
      dma16(ra, St + (C::kALoads * wave + c) * 1024, va[c], (uint32_t)ks * kARow);
    } else if (c < C::kALoads + C::kWLoads) {
      const int j = c - C::kALoads;
      dma16(rw, St + C::kABytes + (C::kWLoads * wave + j) * 1024, vw[j], (uint32_t)ks * C::kWRow);
    } else {
      // the stage's 64 scales, copied whole by every wave (the same bytes to the
      // same place): a per-lane condition here would split the stage's code at a
      // divergent branch, and the scale broadcasts of the decode are then no
      // longer folded into their multiplies
      dma4(rs, St + C::kABytes + C::kWBytes, (uint32_t)lane * 4u, (uint32_t)ks * 256u);
    }
  };
  // weight fragment j as read from LDS (codes: 16 bytes; bf16: 2 x 16 bytes)
  auto read_w = [&](const uint8_t* St, int j) {
    v8i r;
    if (FROM_CODES) {
      const v4i v = *reinterpret_cast<const v4i*>(St + w_rd[0] + j * 1024);
      r = (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
    } else {
      const v4i lo = *reinterpret_cast<const v4i*>(St + w_rd[0] + j * 2048);
      const v4i hi = *reinterpret_cast<const v4i*>(St + w_rd[1] + j * 2048);
      r = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    return r;
  };
  auto read_s = [&](const uint8_t* St) {
    return FROM_CODES ? *reinterpret_cast<const float*>(St + s_rd) : 0.f;
  };
  // raw fragment -> the two MFMA operands (halves n = 0..7 and 8..15 of the lane's 16)
  auto convert = [&](float srow, const v8i& r, v4i* w) {
    if (FROM_CODES) {
      // opaque copy: the broadcasts stay inside this fragment's multiplies
      // instead of being hoisted into 16 extra moves shared by the fragments
      asm volatile("" : "+v"(srow));
      w[0] = deq8<0>((uint32_t)r[0], (uint32_t)r[1], srow);
      w[1] = deq8<1>((uint32_t)r[2], (uint32_t)r[3], srow);
    } else {
      w[0] = (v4i){r[0], r[1], r[2], r[3]};
      w[1] = (v4i){r[4], r[5], r[6], r[7]};
    }
  };

  v4f acc[FBK][NJ];
#pragma unroll
  for (int f = 0; f < FBK; ++f)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int nk = N / BKN;
  auto slot = [&](int s) { return smem + (s % S) * C::kStage; };

  // ---- prologue: stages 0 .. S-2 in flight, stage 0 landed and its operands in registers
#pragma unroll
  for (int c = 0; c < C::kLoads; ++c) issue_one(slot(0), 0, c);
  if (nk > 1) {
#pragma unroll
    for (int c = 0; c < C::kLoads; ++c) issue_one(slot(1), 1, c);
    wait_vmem_lds<C::kLoads>();
  } else {
    wait_vmem_lds<0>();
  }
  barrier_only();
  // A wave whose BM/2 rows all lie past the tile's last valid row (an
  // expert's short last tile) skips its operand reads, conversions and
  // MFMAs; it still issues its share of the copies and joins every barrier.
  // The two waves of a SIMD own the tile's two row halves, so a tile of at
  // most BM/2 valid rows keeps one wave's work per SIMD.
  const bool active = wm * (BM / 2) < rows;
  // FINE (codes, 256-row tiles): fragment j+1's codes are decoded one output
  // word per two of fragment j's 16 MFMAs (read two fragments ahead), so the
  // decode sits between the MFMAs instead of after them.
  constexpr bool FINE = FROM_CODES && FBK == 8;
  v4i a[FBK][2];
  v4i wcur[2];
  v8i rawn;           // FINE: the codes of the next fragment, as read
  float scur = 0.f, sn = 0.f;
  if (active) {
#pragma unroll
    for (int f = 0; f < FBK; ++f)
#pragma unroll
      for (int s = 0; s < 2; ++s) a[f][s] = *reinterpret_cast<const v4i*>(slot(0) + a_rd[s] + f * 2048);
    scur = read_s(slot(0));
    convert(scur, read_w(slot(0), 0), wcur);
    if (FINE) rawn = read_w(slot(0), 1);
  }

  static_assert(S == 3, "the copy slot must differ from the two slots read in a stage");
  // One stage.  ISSUE: copy stage ks+2 into `wr` (the slot of stage ks-1,
  // which no wave reads after the previous barrier); MORE: stage ks+1 (slot
  // `rn`) exists: the barrier before the last fragment makes sure it has
  // landed, then its first weight fragment and its dout operand are read;
  // ACT: the wave computes (see above).  `wr` is distinct from `rd`/`rn`;
  // marking the slots __restrict__ tells the compiler the reads cannot depend
  // on the copies issued here, so it adds no wait for them (the explicit wait
  // + barrier order the ring).
  auto step = [&](int ks, auto issue_c, auto more_c, auto act_c, uint8_t* __restrict__ wr,
                  const uint8_t* __restrict__ rd, const uint8_t* __restrict__ rn) {
    constexpr bool ISSUE = decltype(issue_c)::value;
    constexpr bool MORE = decltype(more_c)::value;
    constexpr bool ACT = decltype(act_c)::value;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      // pieces counted from the fragment the stage barrier precedes
      prio_by_progress((j - (FINE ? NJ - 2 : NJ - 1) + NJ) % NJ);
      if (ISSUE) {
#pragma unroll
        for (int c = j * C::kLoads / NJ; c < (j + 1) * C::kLoads / NJ; ++c) issue_one(wr, ks + S - 1, c);
      }
      if (MORE && j == NJ - (FINE ? 2 : 1)) {
        // every wave's copy of stage ks+1 has landed and every read of this
        // stage's slot has completed (the copies issued so far in this stage
        // may still be in flight)
        if (ISSUE) wait_vmem_lds<((FINE ? NJ - 1 : NJ) * C::kLoads) / NJ>();
        else wait_vmem_lds<0>();
        barrier_only();
      }
      if constexpr (ACT && FINE) {
        v8i raw2;
        if (j + 2 < NJ) raw2 = read_w(rd, j + 2);
        else if (MORE) {
          raw2 = read_w(rn, j + 2 - NJ);
          if (j + 2 == NJ) sn = read_s(rn);
        }
        const bool conv = j + 1 < NJ || MORE;
        // a fresh copy of the scale per fragment: without it the compiler
        // shares each lane broadcast between the fragments of a stage, and a
        // broadcast with several uses is not folded into its multiply (a
        // v_mov_dpp and a zeroing move per weight instead of none)
        float sconv = j + 1 < NJ ? scur : sn;
        asm volatile("" : "+v"(sconv));
        v4i wnext[2];
        sched_fence();
#pragma unroll
        for (int o = 0; o < 8; ++o) {
#pragma unroll
          for (int mm = 2 * o; mm < 2 * o + 2; ++mm) {
            const int s_ = mm / FBK, f = mm % FBK;
            acc[f][j] = mfma_bf16_16x16x32(as_bf(wcur[s_]), as_bf(a[f][s_]), acc[f][j]);
            if (MORE && j == NJ - 1) a[f][s_] = *reinterpret_cast<const v4i*>(rn + a_rd[s_] + f * 2048);
          }
          if (conv) {
            int w;
            switch (o) {
              case 0: w = deq_word<0>(rawn, sconv); break;
              case 1: w = deq_word<1>(rawn, sconv); break;
              case 2: w = deq_word<2>(rawn, sconv); break;
              case 3: w = deq_word<3>(rawn, sconv); break;
              case 4: w = deq_word<4>(rawn, sconv); break;
              case 5: w = deq_word<5>(rawn, sconv); break;
              case 6: w = deq_word<6>(rawn, sconv); break;
              default: w = deq_word<7>(rawn, sconv); break;
            }
            wnext[o >> 2][o & 3] = w;
          }
          sched_fence();
        }
        wcur[0] = wnext[0];
        wcur[1] = wnext[1];
        rawn = raw2;
        if (MORE && j == NJ - 1) scur = sn;
      }
      if constexpr (ACT && !FINE) {
        v8i raw;
        float snext = scur;
        if (j + 1 < NJ) raw = read_w(rd, j + 1);
        else if (MORE) { raw = read_w(rn, 0); snext = read_s(rn); }
        sched_fence();
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int f = 0; f < FBK; ++f) {
            acc[f][j] = mfma_bf16_16x16x32(as_bf(wcur[s]), as_bf(a[f][s]), acc[f][j]);
            // last fragment of the stage: a[f][s] is free, refill it from stage ks+1
            if (MORE && j == NJ - 1) a[f][s] = *reinterpret_cast<const v4i*>(rn + a_rd[s] + f * 2048);
          }
        v4i wnext[2];
        if (j + 1 < NJ || MORE) convert(snext, raw, wnext);
        sched_fence();
        wcur[0] = wnext[0];
        wcur[1] = wnext[1];
        scur = snext;
      }
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto run = [&](auto act_c) {
    int ks = 0;
    for (; ks + S - 1 < nk; ++ks) step(ks, T_{}, T_{}, act_c, slot(ks + S - 1), slot(ks), slot(ks + 1));
    if (ks + 1 < nk) { step(ks, F_{}, T_{}, act_c, slot(ks + 2), slot(ks), slot(ks + 1)); ++ks; }
    step(ks, F_{}, F_{}, act_c, slot(ks + 2), slot(ks), slot(ks + 1));
  };
  if (active) run(T_{});
  else run(F_{});
  prio_by_progress<3>();

  // ---- epilogue: lane owns row wm*128 + f*16 + lane%16, columns wn*BN/4 + j*16 + 4*(lane/16) + 0..3
  // Lanes l and l^16 hold the same row, columns 4q..4q+3 and 4q+4..4q+7 (q even)
  // of two adjacent 16-column fragments.  Trading one 8-byte group gives the
  // even-q lane 8 columns of the first fragment and the odd-q lane 8 of the
  // second, so every store is 16 bytes and an instruction writes 64 contiguous
  // bytes of each row (p: the row at the first fragment's column 0).
  static_assert(NJ % 2 == 0, "fragments are stored in pairs");
  auto store_pair = [&](uint16_t* p, const v2i& x0, const v2i& x1) __attribute__((always_inline)) {
    const bool ev = (q & 1) == 0;
    const v2i sv = ev ? x1 : x0;
    const int r0 = __shfl_xor(sv[0], 16), r1 = __shfl_xor(sv[1], 16);
    const v4i v = ev ? (v4i){x0[0], x0[1], r0, r1} : (v4i){r0, r1, x1[0], x1[1]};
    *reinterpret_cast<v4i*>(p + (ev ? 4 * q : 16 + 4 * (q - 1))) = v;
  };
  if (DSWIGLU) {
    // output and pre-activation rows are [gate | up], 2K wide
    const size_t ld = 2 * (size_t)K;
#pragma unroll
    for (int f = 0; f < FBK; ++f) {
      const int ml = wm * (BM / 2) + f * 16 + (lane & 15);
      if (ml < rows) {
        const size_t rb0 = (size_t)(row0 + ml) * ld + nt * BN + wn * (16 * NJ);
        const size_t rb = rb0 + 4 * q;
        v2i gb[NJ], ub[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          gb[j] = *reinterpret_cast<const v2i*>(preact + rb + j * 16);
          ub[j] = *reinterpret_cast<const v2i*>(preact + rb + K + j * 16);
        }
        v2i pg[NJ], pu[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          float dg[4], du[4];
          dswiglu1(acc[f][j][0], bf16_lo(gb[j][0]), bf16_lo(ub[j][0]), dg[0], du[0]);
          dswiglu1(acc[f][j][1], bf16_hi(gb[j][0]), bf16_hi(ub[j][0]), dg[1], du[1]);
          dswiglu1(acc[f][j][2], bf16_lo(gb[j][1]), bf16_lo(ub[j][1]), dg[2], du[2]);
          dswiglu1(acc[f][j][3], bf16_hi(gb[j][1]), bf16_hi(ub[j][1]), dg[3], du[3]);
          pg[j][0] = (int)pack_bf16x2(dg[0], dg[1]);
          pg[j][1] = (int)pack_bf16x2(dg[2], dg[3]);
          pu[j][0] = (int)pack_bf16x2(du[0], du[1]);
          pu[j][1] = (int)pack_bf16x2(du[2], du[3]);
        }
#pragma unroll
        for (int j = 0; j < NJ; j += 2) {
          store_pair(dlhs + rb0 + j * 16, pg[j], pg[j + 1]);
          store_pair(dlhs + rb0 + K + j * 16, pu[j], pu[j + 1]);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int f = 0; f < FBK; ++f) {
    const int ml = wm * (BM / 2) + f * 16 + (lane & 15);
    if (ml < rows) {
      uint16_t* orow = dlhs + (size_t)(row0 + ml) * K + nt * BN + wn * (16 * NJ);
      v2i pk[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        pk[j][0] = (int)pack_bf16x2(acc[f][j][0], acc[f][j][1]);
        pk[j][1] = (int)pack_bf16x2(acc[f][j][2], acc[f][j][3]);
      }
#pragma unroll
      for (int j = 0; j < NJ; j += 2) store_pair(orow + j * 16, pk[j], pk[j + 1]);
    }
  }
}

// ---------------------------------------------------------------- cached weight block
//
// When the whole contraction of a k-tile fits the LDS as bf16 (BN output
// columns x N contraction values), the block decodes that weight block once
// and reuses it for every row of its chunk of the expert: the MI355X form of
// the single-K-tile cache ("MoE: native FP8 QAT for routed-expert GMMs",
// Implementation: with one K tile the dequantized block stays in VMEM across
// its m tiles; the conversation page's review thread on the cache).  The
// weight block is the decoded bf16 of dequantize_fp8_codes; it never leaves
// the chip.
//
// A block owns (a chunk of up to chunk_rows rows of one expert, BN output
// columns).  Fill: every thread decodes 16-code groups of the block's BN
// weight rows (exact decode, f32 product with the channel's scale, one bf16
// rounding) into LDS, laid out per 64-value contraction stage as
// [BN rows][64 bf16] with the ring's 16-byte swizzle.  After one barrier the
// LDS is read-only: each wave takes row tasks of RW rows of the chunk in turn
// and runs the whole contraction for them with all BN columns, streaming its
// dout rows from global memory straight into registers, D stages ahead of the
// MFMAs (a buffer range per task: rows past the expert's end are never read,
// a stage past the contraction's end loads zeros without a memory access).
// No ring, no barrier in the main loop, so the waves on a SIMD drift apart
// and cover each other's load latency.
//
// Each lane holds, for MFMA half s of stage ks, the contraction values
// 64 ks + 16 (lane / 16) + 8 s + 0..7 of its weight column and dout row, and
// every accumulator sees the stages in order, half 0 before half 1: the
// operand assignment and order of the ring kernel, so the result is bit for
// bit the ring kernel's (and the bf16 arm's on dequantize_fp8_codes' output).
//
// Why only 128 columns and contractions up to 512: every wave reads its dout
// rows once per k-tile, so a block of BN columns reads dout K / BN times.
// Narrower blocks (to fit a longer contraction) multiply that traffic: 32
// columns at a contraction of 2048 (the pages' microbenchmark wi dLHS) read
// dout 128 times and ran 4x slower than the ring kernel, which reads it K/256
// times and decodes each weight tile once per 256 rows.  A 128-column block
// reads dout twice as often as the ring but decodes each weight element once
// per chunk of up to 2048 rows.
constexpr int kCacheMax = 128 * 1024;             // LDS bytes of the cached block

template <int BN>
struct CacheCfg {
  static constexpr int RW = 64;                  // rows per wave task
  static constexpr int FBK = RW / 16;            // 16-row fragments per task
  static constexpr int NJ = BN / 16;             // 16-column fragments (every column of the block)
  static constexpr int D = 1;                    // dout stages in flight ahead of the MFMAs
  static_assert(kCacheMax + sizeof(int) * (3 * kMaxGroups + 1) <= 160 * 1024, "cache + expert table fit the LDS");
};

template <int BN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void gmm_dlhs_cached_kernel(const uint16_t* __restrict__ dout, const uint8_t* __restrict__ codes,
                            const float* __restrict__ wscale, const int* __restrict__ group_sizes, int G, int M,
                            int K, int N, int chunk_rows, uint16_t* __restrict__ dlhs, int* status) {
  using C = CacheCfg<BN>;
  constexpr int FBK = C::FBK, NJ = C::NJ, RW = C::RW, D = C::D;
  constexpr int kStageBytes = BN * kARow;        // one contraction stage of the block: [BN][64] bf16
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int nk = N / BKN;
  int* t_start = reinterpret_cast<int*>(smem + nk * kStageBytes);
  int* t_end = t_start + G;
  int* t_pre = t_end + G;

  build_group_table(group_sizes, G, M, chunk_rows, GroupTable{t_start, t_end, t_pre}, status);
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k_tiles = K / BN;
  const int T = t_pre[G];
  if ((int)blockIdx.x >= T * k_tiles) return;
  // groups of kGroupM chunks walk the k-tiles, chunk fastest (one chunk's rows per XCD)
  int ct, kt;
  raster_tile<kGroupM>(blockIdx.x, T, k_tiles, ct, kt);
  kt = __builtin_amdgcn_readfirstlane(kt);
  const int g = __builtin_amdgcn_readfirstlane(find_group(t_pre, G, ct));
  const int row0 = __builtin_amdgcn_readfirstlane(t_start[g] + (ct - t_pre[g]) * chunk_rows);
  const int rows = __builtin_amdgcn_readfirstlane(min(chunk_rows, t_end[g] - row0));

  // ---- fill: weight rows kt*BN .. kt*BN+BN-1 over the whole contraction, decoded once
  {
    const uint8_t* cg = codes + ((size_t)g * K + (size_t)kt * BN) * N;
    const float* sg = wscale + (size_t)g * N;
    const int nu = N >> 4;                        // 16-value groups per weight row
    for (int t = tid; t < BN * nu; t += kThreads) {
      const int c = t / nu, u = t - c * nu;
      const v4i w = *reinterpret_cast<const v4i*>(cg + (size_t)c * N + 16 * u);
      const v4f* sp = reinterpret_cast<const v4f*>(sg + 16 * u);
      v4i o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint32_t word = (uint32_t)w[2 * h + p];
          const v4f sc = sp[2 * h + p];
          const v2f lo = dec_e4m3x2<false>(word), hi = dec_e4m3x2<true>(word);
          o[h][2 * p] = (int)pack_bf16x2(lo[0] * sc[0], lo[1] * sc[1]);
          o[h][2 * p + 1] = (int)pack_bf16x2(hi[0] * sc[2], hi[1] * sc[3]);
        }
      uint8_t* st = smem + (u >> 2) * kStageBytes;   // stage of these 16 values
      const int ch = (u & 3) * 2;                    // their first 8-value chunk in the stage
      *reinterpret_cast<v4i*>(st + a_swz(c, ch)) = o[0];
      *reinterpret_cast<v4i*>(st + a_swz(c, ch + 1)) = o[1];
    }
  }
  __syncthreads();

  // ---- row tasks: wave w takes tasks w, w + 8, ... of the chunk
  const int q = lane >> 4;
  int w_rd[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) w_rd[s] = a_swz(lane & 15, 2 * q + s);   // + j * 2048 (+ ks * kStageBytes)
  const int ntask = (rows + RW - 1) / RW;
  // Lanes l and l^16 hold the same row, columns 4q..4q+3 and 4q+4..4q+7 (q
  // even) of two adjacent 16-column fragments: trading one 8-byte group makes
  // every store 16 bytes (as in the ring kernel's epilogue).
  auto store_pair = [&](uint16_t* p, const v2i& x0, const v2i& x1) __attribute__((always_inline)) {
    const bool ev = (q & 1) == 0;
    const v2i sv = ev ? x1 : x0;
    const int r0 = __shfl_xor(sv[0], 16), r1 = __shfl_xor(sv[1], 16);
    const v4i v = ev ? (v4i){x0[0], x0[1], r0, r1} : (v4i){r0, r1, x1[0], x1[1]};
    *reinterpret_cast<v4i*>(p + (ev ? 4 * q : 16 + 4 * (q - 1))) = v;
  };
  for (int task = wave; task < ntask; task += kThreads / 64) {
    const int tr0 = row0 + task * RW;
    const int trows = min(RW, rows - task * RW);
    // this task's rows of dout; a load at or past the range's end returns zeros
    const BufRsrc rd = make_rsrc(dout + (size_t)tr0 * N, (uint32_t)trows * (uint32_t)N * 2u);
    uint32_t voff[FBK];
#pragma unroll
    for (int f = 0; f < FBK; ++f)
      voff[f] = (uint32_t)min(16 * f + (lane & 15), trows - 1) * (uint32_t)N * 2u + 32u * (uint32_t)q;
    const uint32_t kPast = 1u << 31;             // a stage offset past the range: no memory access
    auto load = [&](v4i (&b)[FBK][2], int ks) __attribute__((always_inline)) {
      const uint32_t so = ks < nk ? (uint32_t)ks * (uint32_t)kARow : kPast;
#pragma unroll
      for (int f = 0; f < FBK; ++f)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          b[f][s] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rd, voff[f] + 16u * s, so, 0));
    };
    v4f acc[FBK][NJ];
#pragma unroll
    for (int f = 0; f < FBK; ++f)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const v4i (&b)[FBK][2], int ks) __attribute__((always_inline)) {
      const uint8_t* st = smem + ks * kStageBytes;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const v4i w0 = *reinterpret_cast<const v4i*>(st + j * 2048 + w_rd[0]);
        const v4i w1 = *reinterpret_cast<const v4i*>(st + j * 2048 + w_rd[1]);
#pragma unroll
        for (int f = 0; f < FBK; ++f) acc[f][j] = mfma_bf16_16x16x32(as_bf(w0), as_bf(b[f][0]), acc[f][j]);
#pragma unroll
        for (int f = 0; f < FBK; ++f) acc[f][j] = mfma_bf16_16x16x32(as_bf(w1), as_bf(b[f][1]), acc[f][j]);
      }
    };
    // Two register buffers, unrolled so that each is named at compile time.
    // The loop body has no branch (a load whose only use sits behind a branch
    // gets sunk into it, next to its wait); a load past the contraction's end
    // loads nothing, and the odd last stage runs after the loop.  The fences
    // keep each load ahead of the MFMAs it overlaps.
    static_assert(D == 1, "one stage of dout in flight");
    v4i b0[FBK][2], b1[FBK][2];
    load(b0, 0);
    sched_fence();
    int ks = 0;
    for (; ks + 1 < nk; ks += 2) {
      load(b1, ks + 1);
      sched_fence();
      compute(b0, ks);
      sched_fence();
      load(b0, ks + 2);
      sched_fence();
      compute(b1, ks + 1);
      sched_fence();
    }
    if (ks < nk) compute(b0, ks);
    // ---- epilogue: lane owns row tr0 + 16 f + lane%16, columns kt*BN + 16 j + 4 q + 0..3
#pragma unroll
    for (int f = 0; f < FBK; ++f) {
      const int ml = 16 * f + (lane & 15);
      if (ml < trows) {
        uint16_t* orow = dlhs + (size_t)(tr0 + ml) * K + (size_t)kt * BN;
        v2i pk[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          pk[j][0] = (int)pack_bf16x2(acc[f][j][0], acc[f][j][1]);
          pk[j][1] = (int)pack_bf16x2(acc[f][j][2], acc[f][j][3]);
        }
#pragma unroll
        for (int j = 0; j < NJ; j += 2) store_pair(orow + j * 16, pk[j], pk[j + 1]);
      }
    }
  }
}

// The cached block's column width for contraction N (0: the ring kernel).
int cached_bn(int N) { return 2 * 128 * N <= kCacheMax ? 128 : 0; }

template <int BN>
hipError_t launch_dlhs_cached(const uint16_t* dout, const uint8_t* codes, const float* scale, const int* group_sizes,
                              int G, int M, int K, int N, uint16_t* dlhs, int* status, hipStream_t stream) {
  // rows per block: the largest of 2048 / 1024 / 512 / 256 that still gives two blocks per CU
  const long long k_tiles = K / BN;
  const long long want = 2LL * device_cu_count();
  int chunk = 256;
  for (int c : {2048, 1024, 512}) {
    if (((long long)M / c + G) * k_tiles >= want) {
      chunk = c;
      break;
    }
  }
  const long long grid = ((long long)(M + chunk - 1) / chunk + G) * k_tiles;
  const size_t lds = (size_t)2 * BN * N + sizeof(int) * (3 * (size_t)G + 1);
  hipLaunchKernelGGL((gmm_dlhs_cached_kernel<BN>), dim3((unsigned)grid), dim3(kThreads), lds, stream, dout, codes,
                     scale, group_sizes, G, M, K, N, chunk, dlhs, status);
  return hipGetLastError();
}

template <bool FROM_CODES, bool DSWIGLU, int BM>
hipError_t launch_dlhs_bm(const uint16_t* dout, const uint8_t* codes, const float* scale, const uint16_t* wbf16,
                          const int* group_sizes, int G, int M, int K, int N, const uint16_t* preact, uint16_t* dlhs,
                          int* status, hipStream_t stream) {
  const long long max_m_tiles = (M + BM - 1) / BM + G;
  const size_t table = sizeof(int) * (3 * (size_t)G + 1);
  // bf16 weights always take 128-column tiles (a 256-column bf16 ring does not fit the LDS)
  if constexpr (FROM_CODES) {
    if (K % 256 == 0) {
      hipLaunchKernelGGL((gmm_dlhs_kernel<FROM_CODES, 256, DSWIGLU, BM>), dim3((unsigned)(max_m_tiles * (K / 256))),
                         dim3(kThreads), (Cfg<FROM_CODES, 256, BM>::kLds + table), stream, dout, codes, scale, wbf16,
                         group_sizes, G, M, K, N, preact, dlhs, status);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gmm_dlhs_kernel<FROM_CODES, 128, DSWIGLU, BM>), dim3((unsigned)(max_m_tiles * (K / 128))),
                     dim3(kThreads), (Cfg<FROM_CODES, 128, BM>::kLds + table), stream, dout, codes, scale, wbf16,
                     group_sizes, G, M, K, N, preact, dlhs, status);
  return hipGetLastError();
}

template <bool FROM_CODES, bool DSWIGLU>
hipError_t launch_dlhs_impl(const uint16_t* dout, const uint8_t* codes, const float* scale, const uint16_t* wbf16,
                            const int* group_sizes, int G, int M, int K, int N, const uint16_t* preact,
                            uint16_t* dlhs, int* status, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  // the whole contraction of a k-tile fits the LDS: decode each weight block once per chunk of rows
  if constexpr (FROM_CODES && !DSWIGLU) {
    if (cached_bn(N) == 128)
      return launch_dlhs_cached<128>(dout, codes, scale, group_sizes, G, M, K, N, dlhs, status, stream);
  }
  // skinny groups (at most 64 rows per expert on average): 64-row tiles
  if ((long long)M <= 64LL * G)
    return launch_dlhs_bm<FROM_CODES, DSWIGLU, 64>(dout, codes, scale, wbf16, group_sizes, G, M, K, N, preact, dlhs,
                                                  status, stream);
  return launch_dlhs_bm<FROM_CODES, DSWIGLU, 256>(dout, codes, scale, wbf16, group_sizes, G, M, K, N, preact, dlhs,
                                                 status, stream);
}

}  // namespace

hipError_t launch_gmm_dlhs_fp8(const uint16_t* dout, const uint8_t* codes, const float* scale, const int* group_sizes,
                               int G, int M, int K, int N, uint16_t* dlhs, int* status, hipStream_t stream) {
  return launch_dlhs_impl<true, false>(dout, codes, scale, nullptr, group_sizes, G, M, K, N, nullptr, dlhs, status,
                                       stream);
}

hipError_t launch_gmm_dswiglu_fp8(const uint16_t* dout, const uint8_t* codes, const float* scale,
                                  const int* group_sizes, int G, int M, int K, int N, const uint16_t* preact,
                                  uint16_t* d_preact, int* status, hipStream_t stream) {
  return launch_dlhs_impl<true, true>(dout, codes, scale, nullptr, group_sizes, G, M, K, N, preact, d_preact, status,
                                      stream);
}

hipError_t launch_gmm_bf16_dlhs(const uint16_t* dout, const uint16_t* w, const int* group_sizes, int G, int M, int K,
                                int N, uint16_t* dlhs, int* status, hipStream_t stream) {
  return launch_dlhs_impl<false, false>(dout, nullptr, nullptr, w, group_sizes, G, M, K, N, nullptr, dlhs, status,
                                        stream);
}

}  // namespace fp8gmm

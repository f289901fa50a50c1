// Device-side building blocks shared by the kernels of the FP8 grouped matmul:
// vector types, bf16 packing, MFMA wrappers, LDS transpose reads, wave
// reductions and the group_sizes-driven tile schedule.
//
// Target: CDNA4 (gfx950) only, wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gmm {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Status bits raised on the device (kept in the caller's dev_status word).
constexpr int kDevSumClamped = 1;
constexpr int kDevNegativeSize = 2;

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;
constexpr float kAmaxFloor = 1e-12f;

// ----------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Round-to-nearest-even f32 -> bf16 bits, two at a time (one packed
// hardware conversion on gfx950; lo lands in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(((v2f){lo, hi}), v2bf));
}

// ----------------------------------------------------------------- fp8

// Saturating round-to-nearest-even f32 -> e4m3fn code.  The conversion
// instruction rounds to nearest even but turns out-of-range values into
// NaN, so the value is clamped to the largest finite magnitude first.
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
  c = __builtin_fminf(__builtin_fmaxf(c, -kE4M3Max), kE4M3Max);
  d = __builtin_fminf(__builtin_fmaxf(d, -kE4M3Max), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t cvt_e5m2x4(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kE5M2Max), kE5M2Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kE5M2Max), kE5M2Max);
  c = __builtin_fminf(__builtin_fmaxf(c, -kE5M2Max), kE5M2Max);
  d = __builtin_fminf(__builtin_fmaxf(d, -kE5M2Max), kE5M2Max);
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Exact decode of two e4m3fn codes (bytes 0,1 or, with HI, bytes 2,3 of w).
template <bool HI>
__device__ __forceinline__ v2f dec_e4m3x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}
template <bool HI>
__device__ __forceinline__ v2f dec_e5m2x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
}

// ----------------------------------------------------------------- MFMA

// D = A(16x128 e4m3) * B(128x16 e4m3) + C, f32 accumulate.  Lane l holds
// row l%16 of A (column l%16 of B) and the 32 k-values (l/16)*32 + 0..31.
// Zero scale operands select the unscaled instruction.
__device__ __forceinline__ v4f mfma_e4m3_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D = A(32x64 e4m3) * B(64x32 e4m3) + C, f32 accumulate.  Lane l holds row
// l%32 of A (column l%32 of B) and the 32 k-values (l/32)*32 + 0..31; D: lane
// l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
__device__ __forceinline__ v16f mfma_e4m3_32x32x64(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D = A(16x32 bf16) * B(32x16 bf16) + C; lane l holds row l%16 of A (column
// l%16 of B) and k-values (l/16)*8 + 0..7.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x16 bf16) * B(16x32 bf16) + C; lane l holds row l%32 of A and
// k-values (l/32)*8 + 0..7; D: lane l holds column l%32, rows
// 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ----------------------------------------------------------------- LDS

// Transposing 8-byte LDS read (gfx950).  Within each group of 16 lanes, lane
// i receives byte j from address addr[2j + (i>>3)] + (i & 7), where addr[L] is
// the address supplied by lane L of the group.  Supplying
// addr[L] = &T[k0 + L/2][n0 + 8*(L%2)] of a row-major byte tile T hands lane
// i the column T[k0 + 0..7][n0 + i].
__device__ __forceinline__ v2i lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(v2i, const_cast<void*>(p)));
}

// ----------------------------------------------------------------- global -> LDS copies

typedef __amdgpu_buffer_rsrc_t BufRsrc;

constexpr int kCpolStream = 2;   // buffer-load cache policy: streaming (non-temporal)

// Raw buffer resource over [base, base + bytes); loads at or past the end
// return zeros instead of touching memory.
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One 16-byte chunk per lane from buffer offset voff + soff straight into LDS:
// lane i's chunk lands at lds_wave_base + 16*i (lds_wave_base is wave-uniform).
__device__ __forceinline__ void dma16(BufRsrc r, void* lds_wave_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds_wave_base), 16, voff, soff, 0, 0);
}

// Wait until every vector memory operation of this wave has completed
// (s_waitcnt vmcnt(0); the other counters are left alone).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One dword per lane: lane i's value lands at lds_wave_base + 4*i.
__device__ __forceinline__ void dma4(BufRsrc r, void* lds_wave_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds_wave_base), 4, voff, soff, 0, 0);
}

// Wait until at most N vector memory operations of this wave are outstanding
// (they complete in issue order, so the older ones have landed) and every LDS
// operation has completed: s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N>
__device__ __forceinline__ void wait_vmem_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
  asm volatile("" ::: "memory");   // no load of the landed data may be hoisted above the wait
}

// x / s for the quantizers, from r = 1/s (correctly rounded, one division per
// scale): q0 = x*r, the negated residual q0*s - x (exact through the fma) and
// one correction.  Negating the residual keeps the sign of a zero x through
// the last fma (-0 stays -0) without a copysign; the result has the same bits
// as copysign(fma(x - q0*s, r, q0), x).  Over the quantizers' inputs -- x a
// bf16 value with |x| <= amax, s = f32(max(amax, 1e-12) / FMAX), FMAX 448 or
// 57344, amax finite -- the result equals the IEEE quotient wherever the
// quotient is at least half the smallest subnormal code of the format (below
// that both encode to zero): tests/test_div_by_scale.py checks every such pair
// (and the equality with the copysign form).  s must be finite; callers divide
// directly otherwise.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float q0 = x * r;
  const float en = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-en, r, q0);
}

// Workgroup barrier without the memory fence of __syncthreads(): it does not
// wait for this wave's outstanding LDS-destination loads, which is what lets
// a copy two stages ahead stay in flight.  Callers wait for what they need
// (wait_vmem_lds) before it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scheduling fence: the compiler may not move instructions across it, so a
// prefetch stays ahead of the MFMAs it is meant to overlap.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Issue priority by progress.  The two waves of a SIMD leave each stage
// barrier together, and among waves of equal priority the sequencer issues
// the older one first, so the younger wave ends every stage alone and the
// older one waits for it at the next barrier (measured on the tgmm: the
// younger waves' stage bodies took 1.5x as long).  A loop body in P pieces
// between two barriers calls this at the start of piece P (0 = just past the
// barrier): the wave that is behind gets the higher priority, which keeps the
// two waves within about one piece of each other.  Priority 0 is restored
// after the loop.
template <int P>
__device__ __forceinline__ void prio_by_progress() {
  static_assert(P >= 0, "piece index");
  if constexpr (P == 0) __builtin_amdgcn_s_setprio(3);
  else if constexpr (P == 1) __builtin_amdgcn_s_setprio(2);
  else if constexpr (P == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// The same for a piece index known only after unrolling (p < 4 selects the
// level, larger values take priority 0).
__device__ __forceinline__ void prio_by_progress(int p) {
  switch (p) {
    case 0: prio_by_progress<0>(); break;
    case 1: prio_by_progress<1>(); break;
    case 2: prio_by_progress<2>(); break;
    default: prio_by_progress<3>(); break;
  }
}

// Ask the scheduler for a group of `n` instructions of the classes in `mask`
// (0x2 VALU, 0x8 MFMA, 0x100 LDS read, 0x20 VMEM read) at this point of the
// sequence; consecutive calls with the same id interleave the classes.
#define SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// ----------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// ----------------------------------------------------------------- schedule

// Number of valid rows: sum of max(size, 0), clamped to M.  Computed by one
// wave; every lane returns the same value.  The host guarantees M < 2^24, so
// the clamped partial sums never overflow.
__device__ __forceinline__ int valid_rows(const int* __restrict__ group_sizes, int G, int M) {
  const int lane = threadIdx.x & 63;
  int s = 0;
  for (int g = lane; g < G; g += 64) s = min(s + min(max(group_sizes[g], 0), M), M);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s = min(s + __shfl_xor(s, o, 64), M);
  return s;
}

// Group table in LDS: for each expert g, its valid rows [start, end) and the
// exclusive prefix of its m-tile count (tiles of `bm` rows aligned to the
// expert's first row).  Built by wave 0; the caller synchronises.
struct GroupTable {
  int* start;   // [G]
  int* end;     // [G]
  int* tpre;    // [G + 1]
};

__device__ __forceinline__ void build_group_table(const int* __restrict__ group_sizes, int G, int M, int bm,
                                                  GroupTable t, int* status) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int row_carry = 0, tile_carry = 0;
  int flags = 0;
  for (int base = 0; base < G; base += 64) {
    int g = base + lane;
    int raw = g < G ? group_sizes[g] : 0;
    if (raw < 0) flags |= kDevNegativeSize;
    if (raw > M) flags |= kDevSumClamped;
    int sz = min(max(raw, 0), M);                     // M < 2^24: no overflow below
    int incl = wave_incl_scan(sz);
    int e_raw = row_carry + incl;                     // may exceed M before clamping
    int s_raw = e_raw - sz;
    int st = min(s_raw, M), en = min(e_raw, M);
    if (e_raw > M && sz > 0) flags |= kDevSumClamped;
    int nt = (en - st + bm - 1) / bm;
    int tincl = wave_incl_scan(nt);
    if (g < G) {
      t.start[g] = st;
      t.end[g] = en;
      t.tpre[g] = tile_carry + tincl - nt;
    }
    row_carry = min(__shfl(e_raw, 63, 64), M);
    tile_carry += __shfl(tincl, 63, 64);
  }
  if (lane == 0) t.tpre[G] = tile_carry;
  int any = flags;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) any |= __shfl_xor(any, o, 64);
  if (status != nullptr && lane == 0 && blockIdx.x == 0 && blockIdx.y == 0 && any) atomicOr(status, any);
}

// Expert owning global m-tile `mt` (binary search over the tile prefix).
__device__ __forceinline__ int find_group(const int* tpre, int G, int mt) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (tpre[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Logical tile of block b in the m-grouped raster of the GEMMs: groups of
// kGroupM m-tiles walk the n-tiles, m fastest.  Blocks are dispatched
// round-robin over the 8 XCDs, so with kGroupM = 8 each XCD takes one m-tile
// of a group through all its n-tiles and keeps that tile's rows in its own
// L2 (the weights come from the MALL).  Measured on the bench GEMMs, this
// beat a remap that gives each XCD a contiguous range of logical tiles by
// 2-6 %.
template <int kGroupM>
__device__ __forceinline__ void raster_tile(int b, int T, int n_tiles, int& mt, int& nt) {
  const int width = kGroupM * n_tiles;
  const int first_m = (b / width) * kGroupM;
  const int gsz = min(T - first_m, kGroupM);
  mt = first_m + (b % width) % gsz;
  nt = (b % width) / gsz;
}

}  // namespace fp8gmm

// C ABI of the library: argument validation, workspace layout and kernel
// launches on the caller's stream.  Declarations and the contract of every
// entry point are in include/fp8_moe_grouped.h.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/fp8_moe_grouped.h"
#include "launch.hpp"

using namespace fp8gmm;

// Scratch of gmm_fp8_fwd_noalloc: the activation codes and row scales that
// gmm_fp8_fwd keeps in the caller's workspace.  Every GPU the library runs on
// holds its own copy until the process ends.  Host code never uses this name
// as an address (on the host it is only a stand-in): the device address comes
// from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[FP8GMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int64_t M, int64_t K, int64_t N, int32_t G) {
  if (M < 0 || M > kMaxRows || K <= 0 || N <= 0 || G <= 0) return FP8GMM_ERR_SHAPE;
  if (G > kMaxGroups) return FP8GMM_ERR_UNSUPPORTED;
  if (K % 128 != 0 || N % 128 != 0) return FP8GMM_ERR_UNSUPPORTED;
  if ((long long)G * K * N >= (1LL << 40)) return FP8GMM_ERR_SHAPE;
  if ((long long)K * N >= (1LL << 31)) return FP8GMM_ERR_UNSUPPORTED;   // one expert's codes per buffer range
  return FP8GMM_OK;
}

// Forward workspace: activation codes [M, K] then row scales [M].
size_t fwd_ws(int64_t M, int64_t K) { return align_up((size_t)M * K) + align_up((size_t)M * 4); }

// Variant forward workspace: codes [M, K] then scales [M, ceil(K/512)] (or [M]).
size_t variant_ws(int64_t M, int64_t K, int32_t lhs_block) {
  const int64_t nb = lhs_block == 512 ? (K + 511) / 512 : 1;
  return align_up((size_t)M * K) + align_up((size_t)M * nb * 4);
}

int fwd_common(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes, int64_t M,
               int64_t K, int64_t N, int32_t G, void* out, void* preact, uint8_t* dbg_codes, float* dbg_scale,
               void* ws, size_t ws_bytes, int32_t* dev_status, void* stream, bool swiglu) {
  if (!codes || !scale || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!lhs || !out)) return FP8GMM_ERR_NULL;
  if (K > kMaxK) return FP8GMM_ERR_UNSUPPORTED;
  if (swiglu && ((N / 2) % 128 != 0)) return FP8GMM_ERR_UNSUPPORTED;
  if (!aligned16(lhs) || !aligned16(codes) || !aligned16(scale) || !aligned16(out) || !aligned16(preact) ||
      (dbg_codes && !aligned16(dbg_codes)))
    return FP8GMM_ERR_ALIGN;   // NULL (M == 0) counts as aligned
  const size_t need = fwd_ws(M, K);
  if (M > 0 && (!ws || ws_bytes < need)) return FP8GMM_ERR_WORKSPACE;
  if (M == 0) return FP8GMM_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* aq = dbg_codes ? dbg_codes : static_cast<uint8_t*>(ws);
  float* as = dbg_scale ? dbg_scale : reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align_up((size_t)M * K));
  if (launch_quant_rows_e4m3(static_cast<const uint16_t*>(lhs), group_sizes, G, (int)M, (int)K, aq, as, s) !=
      hipSuccess)
    return FP8GMM_ERR_HIP;
  if (launch_gmm_fp8_fwd(aq, as, codes, scale, group_sizes, G, (int)M, (int)K, (int)N, swiglu,
                         static_cast<uint16_t*>(out), static_cast<uint16_t*>(preact), dev_status, s) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

}  // namespace

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device id

// Device address of the current device's scratch (looked up on the first call
// on each device; a race between two first calls stores the same address).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8GMM_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FP8GMM_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FP8GMM_OK;
}

}  // namespace

extern "C" {

int gmm_fp8_fwd(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes, int64_t M,
                int64_t K, int64_t N, int32_t G, void* out, uint8_t* dbg_codes, float* dbg_scale, void* ws,
                size_t ws_bytes, int32_t* dev_status, void* stream) {
  return fwd_common(lhs, codes, scale, group_sizes, M, K, N, G, out, nullptr, dbg_codes, dbg_scale, ws, ws_bytes,
                    dev_status, stream, false);
}

int gmm_fp8_fwd_noalloc(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                        int64_t M, int64_t K, int64_t N, int32_t G, void* out, int32_t* dev_status, void* stream) {
  if (!codes || !scale || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!lhs || !out)) return FP8GMM_ERR_NULL;
  if (K > kMaxK) return FP8GMM_ERR_UNSUPPORTED;
  if (!aligned16(lhs) || !aligned16(codes) || !aligned16(scale) || !aligned16(out)) return FP8GMM_ERR_ALIGN;
  if (fwd_ws(M, K) > FP8GMM_NOALLOC_SCRATCH_BYTES) return FP8GMM_ERR_SCRATCH;
  if (M == 0) return FP8GMM_OK;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != FP8GMM_OK) return st;
  return fwd_common(lhs, codes, scale, group_sizes, M, K, N, G, out, nullptr, nullptr, nullptr, ws,
                    FP8GMM_NOALLOC_SCRATCH_BYTES, dev_status, stream, false);
}

int gmm_silu_fp8(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes, int64_t M,
                 int64_t K, int64_t N, int32_t G, void* out, void* preact, uint8_t* dbg_codes, float* dbg_scale,
                 void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  return fwd_common(lhs, codes, scale, group_sizes, M, K, N, G, out, preact, dbg_codes, dbg_scale, ws, ws_bytes,
                    dev_status, stream, true);
}

int gmm_fp8_fwd_variant(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                        int64_t M, int64_t K, int64_t N, int32_t G, int32_t lhs_block, int32_t flags, void* out,
                        uint8_t* dbg_codes, float* dbg_scale, void* ws, size_t ws_bytes, int32_t* dev_status,
                        void* stream) {
  if (!codes || !scale || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!lhs || !out)) return FP8GMM_ERR_NULL;
  if (K > kMaxK || (lhs_block != 0 && lhs_block != 512)) return FP8GMM_ERR_UNSUPPORTED;
  if (flags & ~(FP8GMM_LHS_SCALE_BF16 | FP8GMM_ACC_BF16 | FP8GMM_RHS_SCALE_FIRST)) return FP8GMM_ERR_UNSUPPORTED;
  if (!aligned16(lhs) || !aligned16(codes) || !aligned16(scale) || !aligned16(out) ||
      (dbg_codes && !aligned16(dbg_codes)))
    return FP8GMM_ERR_ALIGN;
  const size_t need = variant_ws(M, K, lhs_block);
  if (M > 0 && (!ws || ws_bytes < need)) return FP8GMM_ERR_WORKSPACE;
  if (M == 0) return FP8GMM_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* aq = dbg_codes ? dbg_codes : static_cast<uint8_t*>(ws);
  float* as = dbg_scale ? dbg_scale : reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align_up((size_t)M * K));
  const bool block = lhs_block == 512;
  if (launch_quant_rows_e4m3_variant(static_cast<const uint16_t*>(lhs), group_sizes, G, (int)M, (int)K, block,
                                     (flags & FP8GMM_LHS_SCALE_BF16) != 0, aq, as, s) != hipSuccess ||
      launch_gmm_fp8_fwd_variant(aq, as, codes, scale, group_sizes, G, (int)M, (int)K, (int)N, block,
                                 (flags & FP8GMM_ACC_BF16) != 0, (flags & FP8GMM_RHS_SCALE_FIRST) != 0,
                                 static_cast<uint16_t*>(out), dev_status, s) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

int quantize_rows_fp8(const void* lhs, const int32_t* group_sizes, int64_t M, int64_t K, int32_t G,
                      uint8_t* codes_out, float* scale_out, void* stream) {
  if (!group_sizes) return FP8GMM_ERR_NULL;
  if (M < 0 || M > kMaxRows || K <= 0 || G <= 0) return FP8GMM_ERR_SHAPE;
  if (M > 0 && (!lhs || !codes_out || !scale_out)) return FP8GMM_ERR_NULL;
  if (G > kMaxGroups || K % 128 != 0 || K > kMaxK) return FP8GMM_ERR_UNSUPPORTED;
  if (!aligned16(lhs) || !aligned16(codes_out)) return FP8GMM_ERR_ALIGN;
  if (M == 0) return FP8GMM_OK;
  if (launch_quant_rows_e4m3(static_cast<const uint16_t*>(lhs), group_sizes, G, (int)M, (int)K, codes_out, scale_out,
                             reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

static int fwd_q_common(const uint8_t* aq, const float* ascale, const uint8_t* codes, const float* scale,
                        const int32_t* group_sizes, int64_t M, int64_t K, int64_t N, int32_t G, void* out,
                        void* preact, int32_t* dev_status, void* stream, bool swiglu) {
  if (!codes || !scale || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!aq || !ascale || !out)) return FP8GMM_ERR_NULL;
  if (swiglu && ((N / 2) % 128 != 0)) return FP8GMM_ERR_UNSUPPORTED;
  if (!aligned16(aq) || !aligned16(codes) || !aligned16(scale) || !aligned16(out) || !aligned16(preact))
    return FP8GMM_ERR_ALIGN;
  if (M == 0) return FP8GMM_OK;
  if (launch_gmm_fp8_fwd(aq, ascale, codes, scale, group_sizes, G, (int)M, (int)K, (int)N, swiglu,
                         static_cast<uint16_t*>(out), static_cast<uint16_t*>(preact), dev_status,
                         reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

int gmm_fp8_fwd_q(const uint8_t* aq, const float* ascale, const uint8_t* codes, const float* scale,
                  const int32_t* group_sizes, int64_t M, int64_t K, int64_t N, int32_t G, void* out,
                  int32_t* dev_status, void* stream) {
  return fwd_q_common(aq, ascale, codes, scale, group_sizes, M, K, N, G, out, nullptr, dev_status, stream, false);
}

int gmm_silu_fp8_q(const uint8_t* aq, const float* ascale, const uint8_t* codes, const float* scale,
                   const int32_t* group_sizes, int64_t M, int64_t K, int64_t N, int32_t G, void* out, void* preact,
                   int32_t* dev_status, void* stream) {
  return fwd_q_common(aq, ascale, codes, scale, group_sizes, M, K, N, G, out, preact, dev_status, stream, true);
}

int dequantize_fp8_codes(const uint8_t* codes, const float* scale, int32_t G, int64_t K, int64_t N, void* out,
                         void* stream) {
  if (!codes || !scale || !out) return FP8GMM_ERR_NULL;
  if (G <= 0 || K <= 0 || N <= 0) return FP8GMM_ERR_SHAPE;
  if (N % 16 != 0) return FP8GMM_ERR_UNSUPPORTED;
  if ((long long)G * K * N >= (1LL << 40)) return FP8GMM_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scale) || !aligned16(out)) return FP8GMM_ERR_ALIGN;
  if (launch_dequant(codes, scale, G, K, N, static_cast<uint16_t*>(out), reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

int gmm_dlhs_fp8(const void* dout, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                 int64_t M, int64_t K, int64_t N, int32_t G, void* dlhs, void* ws, size_t ws_bytes,
                 int32_t* dev_status, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!codes || !scale || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!dout || !dlhs)) return FP8GMM_ERR_NULL;
  if (!aligned16(dout) || !aligned16(codes) || !aligned16(scale) || !aligned16(dlhs)) return FP8GMM_ERR_ALIGN;
  if (M == 0) return FP8GMM_OK;
  if (launch_gmm_dlhs_fp8(static_cast<const uint16_t*>(dout), codes, scale, group_sizes, G, (int)M, (int)K, (int)N,
                          static_cast<uint16_t*>(dlhs), dev_status, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

int tgmm_quant(const void* lhs, const void* dout, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
               int32_t G, int32_t grad_dtype, int32_t tile_m, float* drhs, float* dbg_sL, float* dbg_sD, void* ws,
               size_t ws_bytes, int32_t* dev_status, void* stream) {
  if (!group_sizes || !drhs) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!lhs || !dout)) return FP8GMM_ERR_NULL;
  if (grad_dtype != FP8GMM_E4M3 && grad_dtype != FP8GMM_E5M2) return FP8GMM_ERR_UNSUPPORTED;
  if (tile_m != 512) return FP8GMM_ERR_UNSUPPORTED;
  if (!aligned16(lhs) || !aligned16(dout) || !aligned16(drhs) || (dbg_sL && !aligned16(dbg_sL)) ||
      (dbg_sD && !aligned16(dbg_sD)))
    return FP8GMM_ERR_ALIGN;
  const size_t need = tgmm_workspace_bytes(M, K, N, G);
  if (need > 0 && (!ws || ws_bytes < need)) return FP8GMM_ERR_WORKSPACE;
  if (launch_tgmm_quant(static_cast<const uint16_t*>(lhs), static_cast<const uint16_t*>(dout), group_sizes, G,
                        (int)M, (int)K, (int)N, grad_dtype == FP8GMM_E5M2, drhs, dbg_sL, dbg_sD, ws, dev_status,
                        reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

int gmm_dswiglu_fp8(const void* dout, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                    const void* preact, int64_t M, int64_t K, int64_t N, int32_t G, void* d_preact,
                    int32_t* dev_status, void* stream) {
  if (!codes || !scale || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!dout || !preact || !d_preact)) return FP8GMM_ERR_NULL;
  if (!aligned16(dout) || !aligned16(codes) || !aligned16(scale) || !aligned16(preact) || !aligned16(d_preact))
    return FP8GMM_ERR_ALIGN;
  if (M == 0) return FP8GMM_OK;
  if (launch_gmm_dswiglu_fp8(static_cast<const uint16_t*>(dout), codes, scale, group_sizes, G, (int)M, (int)K,
                             (int)N, static_cast<const uint16_t*>(preact), static_cast<uint16_t*>(d_preact),
                             dev_status, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

int tgmm_dense_quant(const void* lhs, const void* dout, const int32_t* group_sizes, int64_t M, int64_t K,
                     int64_t N, int32_t G, int32_t grad_dtype, float* drhs, float* dbg_row_scale,
                     float* dbg_col_scale, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  if (!group_sizes || !drhs) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!lhs || !dout)) return FP8GMM_ERR_NULL;
  if (grad_dtype != FP8GMM_E4M3 && grad_dtype != FP8GMM_E5M2) return FP8GMM_ERR_UNSUPPORTED;
  if (K > kMaxK) return FP8GMM_ERR_UNSUPPORTED;
  if (!aligned16(lhs) || !aligned16(dout) || !aligned16(drhs) || (dbg_col_scale && !aligned16(dbg_col_scale)))
    return FP8GMM_ERR_ALIGN;
  const size_t need = tgmm_dense_workspace_bytes(M, K, N, G);
  if (need > 0 && (!ws || ws_bytes < need)) return FP8GMM_ERR_WORKSPACE;
  if (launch_tgmm_dense(static_cast<const uint16_t*>(lhs), static_cast<const uint16_t*>(dout), group_sizes, G,
                        (int)M, (int)K, (int)N, grad_dtype == FP8GMM_E5M2, drhs, dbg_row_scale, dbg_col_scale, ws,
                        dev_status, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

static int bf16_fwd_common(const void* lhs, const void* w, const int32_t* group_sizes, int64_t M, int64_t K,
                           int64_t N, int32_t G, void* out, int32_t* dev_status, void* stream, bool swiglu) {
  if (!w || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!lhs || !out)) return FP8GMM_ERR_NULL;
  if (swiglu && ((N / 2) % 128 != 0)) return FP8GMM_ERR_UNSUPPORTED;
  if ((long long)K * N * 2 >= (1LL << 32)) return FP8GMM_ERR_UNSUPPORTED;   // one expert's bf16 weight per range
  if (!aligned16(lhs) || !aligned16(w) || !aligned16(out)) return FP8GMM_ERR_ALIGN;
  if (M == 0) return FP8GMM_OK;
  if (launch_gmm_bf16_fwd(static_cast<const uint16_t*>(lhs), static_cast<const uint16_t*>(w), group_sizes, G, (int)M,
                          (int)K, (int)N, swiglu, static_cast<uint16_t*>(out), dev_status,
                          reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

int gmm_bf16_fwd(const void* lhs, const void* w, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
                 int32_t G, void* out, int32_t* dev_status, void* stream) {
  return bf16_fwd_common(lhs, w, group_sizes, M, K, N, G, out, dev_status, stream, false);
}

int gmm_bf16_silu(const void* lhs, const void* w, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
                  int32_t G, void* out, int32_t* dev_status, void* stream) {
  return bf16_fwd_common(lhs, w, group_sizes, M, K, N, G, out, dev_status, stream, true);
}

int gmm_bf16_dlhs(const void* dout, const void* w, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
                  int32_t G, void* dlhs, int32_t* dev_status, void* stream) {
  if (!w || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_common(M, K, N, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!dout || !dlhs)) return FP8GMM_ERR_NULL;
  if (!aligned16(dout) || !aligned16(w) || !aligned16(dlhs)) return FP8GMM_ERR_ALIGN;
  if (M == 0) return FP8GMM_OK;
  if (launch_gmm_bf16_dlhs(static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(w), group_sizes, G,
                           (int)M, (int)K, (int)N, static_cast<uint16_t*>(dlhs), dev_status,
                           reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

// Shapes of one FFN: x [M, H], wi [G, H, 2I], wo [G, I, H].
static int check_ffn(int64_t M, int64_t H, int64_t I, int32_t G) {
  if (H <= 0 || I <= 0) return FP8GMM_ERR_SHAPE;
  int st = check_common(M, H, 2 * I, G);
  if (st != FP8GMM_OK) return st;
  st = check_common(M, I, H, G);
  if (st != FP8GMM_OK) return st;
  if (H > kMaxK || I > kMaxK) return FP8GMM_ERR_UNSUPPORTED;
  return FP8GMM_OK;
}

static size_t ffn_fwd_ws(int64_t M, int64_t H, int64_t I) { return fwd_ws(M, H > I ? H : I); }

static size_t ffn_bwd_ws(int64_t M, int64_t H, int64_t I, int32_t G) {
  const size_t a = tgmm_workspace_bytes(M, I, H, G), b = tgmm_workspace_bytes(M, H, 2 * I, G);
  return a > b ? a : b;
}

int moe_ffn_fp8_fwd(const void* x, const uint8_t* wi_codes, const float* wi_scale, const uint8_t* wo_codes,
                    const float* wo_scale, const int32_t* group_sizes, int64_t M, int64_t H, int64_t I, int32_t G,
                    void* h, void* preact, void* y, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream) {
  if (!wi_codes || !wi_scale || !wo_codes || !wo_scale || !group_sizes) return FP8GMM_ERR_NULL;
  int st = check_ffn(M, H, I, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!x || !h || !y)) return FP8GMM_ERR_NULL;
  if (!aligned16(x) || !aligned16(wi_codes) || !aligned16(wi_scale) || !aligned16(wo_codes) ||
      !aligned16(wo_scale) || !aligned16(h) || !aligned16(preact) || !aligned16(y))
    return FP8GMM_ERR_ALIGN;
  const size_t need = ffn_fwd_ws(M, H, I);
  if (M > 0 && (!ws || ws_bytes < need)) return FP8GMM_ERR_WORKSPACE;
  if (M == 0) return FP8GMM_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the two activation quantizations share the workspace (stream order)
  uint8_t* aq = static_cast<uint8_t*>(ws);
  float* as = reinterpret_cast<float*>(aq + align_up((size_t)M * (size_t)(H > I ? H : I)));
  if (launch_quant_rows_e4m3(static_cast<const uint16_t*>(x), group_sizes, G, (int)M, (int)H, aq, as, s) !=
          hipSuccess ||
      launch_gmm_fp8_fwd(aq, as, wi_codes, wi_scale, group_sizes, G, (int)M, (int)H, (int)(2 * I), true,
                         static_cast<uint16_t*>(h), static_cast<uint16_t*>(preact), dev_status, s) != hipSuccess ||
      launch_quant_rows_e4m3(static_cast<const uint16_t*>(h), group_sizes, G, (int)M, (int)I, aq, as, s) !=
          hipSuccess ||
      launch_gmm_fp8_fwd(aq, as, wo_codes, wo_scale, group_sizes, G, (int)M, (int)I, (int)H, false,
                         static_cast<uint16_t*>(y), nullptr, dev_status, s) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

int moe_ffn_fp8_bwd(const void* x, const void* h, const void* preact, const void* dy, const uint8_t* wi_codes,
                    const float* wi_scale, const uint8_t* wo_codes, const float* wo_scale,
                    const int32_t* group_sizes, int64_t M, int64_t H, int64_t I, int32_t G, int32_t grad_dtype,
                    void* d_preact, void* dx, float* dwi, float* dwo, void* ws, size_t ws_bytes,
                    int32_t* dev_status, void* stream) {
  if (!wi_codes || !wi_scale || !wo_codes || !wo_scale || !group_sizes || !dwi || !dwo) return FP8GMM_ERR_NULL;
  int st = check_ffn(M, H, I, G);
  if (st != FP8GMM_OK) return st;
  if (M > 0 && (!x || !h || !preact || !dy || !d_preact)) return FP8GMM_ERR_NULL;
  if (grad_dtype != FP8GMM_E4M3 && grad_dtype != FP8GMM_E5M2) return FP8GMM_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(h) || !aligned16(preact) || !aligned16(dy) || !aligned16(wi_codes) ||
      !aligned16(wi_scale) || !aligned16(wo_codes) || !aligned16(wo_scale) || !aligned16(d_preact) ||
      !aligned16(dx) || !aligned16(dwi) || !aligned16(dwo))
    return FP8GMM_ERR_ALIGN;
  const size_t need = ffn_bwd_ws(M, H, I, G);
  if (need > 0 && (!ws || ws_bytes < need)) return FP8GMM_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool e5m2 = grad_dtype == FP8GMM_E5M2;
  uint16_t* dz = static_cast<uint16_t*>(d_preact);
  if (M > 0) {
    if (launch_gmm_dswiglu_fp8(static_cast<const uint16_t*>(dy), wo_codes, wo_scale, group_sizes, G, (int)M, (int)I,
                               (int)H, static_cast<const uint16_t*>(preact), dz, dev_status, s) != hipSuccess)
      return FP8GMM_ERR_HIP;
    if (dx && launch_gmm_dlhs_fp8(dz, wi_codes, wi_scale, group_sizes, G, (int)M, (int)H, (int)(2 * I),
                                  static_cast<uint16_t*>(dx), dev_status, s) != hipSuccess)
      return FP8GMM_ERR_HIP;
  }
  // weight gradients (written fully, zeros for experts without rows)
  if (launch_tgmm_quant(static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(dy), group_sizes, G, (int)M,
                        (int)I, (int)H, e5m2, dwo, nullptr, nullptr, ws, dev_status, s) != hipSuccess ||
      launch_tgmm_quant(static_cast<const uint16_t*>(x), dz, group_sizes, G, (int)M, (int)H, (int)(2 * I), e5m2, dwi,
                        nullptr, nullptr, ws, dev_status, s) != hipSuccess)
    return FP8GMM_ERR_HIP;
  return FP8GMM_OK;
}

size_t fp8gmm_workspace_bytes(int32_t op, int64_t M, int64_t K, int64_t N, int32_t G, int32_t tile_m) {
  if (check_common(M, K, N, G) != FP8GMM_OK) return 0;
  switch (op) {
    case FP8GMM_OP_FWD:
    case FP8GMM_OP_SILU:
      return fwd_ws(M, K);
    case FP8GMM_OP_TGMM:
      return tile_m == 512 ? tgmm_workspace_bytes(M, K, N, G) : 0;
    case FP8GMM_OP_TGMM_DENSE:
      return K <= kMaxK ? tgmm_dense_workspace_bytes(M, K, N, G) : 0;
    case FP8GMM_OP_FWD_VARIANT:
      return (tile_m == 0 || tile_m == 512) ? variant_ws(M, K, tile_m) : 0;
    case FP8GMM_OP_FFN_FWD:
      return check_ffn(M, K, N, G) == FP8GMM_OK ? ffn_fwd_ws(M, K, N) : 0;
    case FP8GMM_OP_FFN_BWD:
      return (tile_m == 512 && check_ffn(M, K, N, G) == FP8GMM_OK) ? ffn_bwd_ws(M, K, N, G) : 0;
    default:
      return 0;
  }
}

const char* fp8gmm_status_string(int32_t status) {
  switch (status) {
    case FP8GMM_OK: return "ok";
    case FP8GMM_ERR_NULL: return "a required pointer is NULL";
    case FP8GMM_ERR_SHAPE: return "a size is out of range";
    case FP8GMM_ERR_UNSUPPORTED: return "unsupported shape or option";
    case FP8GMM_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case FP8GMM_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8GMM_ERR_HIP: return "a HIP kernel launch failed";
    case FP8GMM_ERR_SCRATCH: return "the input does not fit the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

}  // extern "C"

// Host-side launchers of the library's kernels (internal; the public C ABI is
// include/fp8_moe_grouped.h).  Every launcher enqueues on `stream`, never
// synchronises and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fp8gmm {

// Largest K handled by the row quantizer (512 bf16 per lane-chunk x 32).
constexpr int kMaxK = 16384;
// Largest number of experts (the group table lives in LDS).
constexpr int kMaxGroups = 1024;
// Largest static row count (keeps the clamped row prefix sums in int32).
constexpr long long kMaxRows = (1LL << 24) - 1;

// Compute units of the current device, looked up once per device id
// (persistent kernels launch one block per CU).
inline int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_quant_rows_e4m3(const uint16_t* lhs, const int* group_sizes, int G, int M, int K,
                                  uint8_t* codes, float* scales, hipStream_t stream);

hipError_t launch_gmm_fp8_fwd(const uint8_t* aq, const float* ascale, const uint8_t* codes, const float* wscale,
                              const int* group_sizes, int G, int M, int K, int N, bool swiglu, uint16_t* out,
                              uint16_t* preact, int* status, hipStream_t stream);

hipError_t launch_gmm_dlhs_fp8(const uint16_t* dout, const uint8_t* codes, const float* scale, const int* group_sizes,
                               int G, int M, int K, int N, uint16_t* dlhs, int* status, hipStream_t stream);

// dLHS with the dSwiGLU epilogue: preact and d_preact are bf16 [M, 2K].
hipError_t launch_gmm_dswiglu_fp8(const uint16_t* dout, const uint8_t* codes, const float* scale,
                                  const int* group_sizes, int G, int M, int K, int N, const uint16_t* preact,
                                  uint16_t* d_preact, int* status, hipStream_t stream);

hipError_t launch_gmm_bf16_dlhs(const uint16_t* dout, const uint16_t* w, const int* group_sizes, int G, int M, int K,
                                int N, uint16_t* dlhs, int* status, hipStream_t stream);

// Ops-level LHS-quantization variants: ascale holds [M, ceil(K/512)] block scales when block512.
hipError_t launch_quant_rows_e4m3_variant(const uint16_t* lhs, const int* group_sizes, int G, int M, int K,
                                          bool block512, bool scale_bf16, uint8_t* codes, float* scales,
                                          hipStream_t stream);
hipError_t launch_gmm_fp8_fwd_variant(const uint8_t* aq, const float* ascale, const uint8_t* codes,
                                      const float* wscale, const int* group_sizes, int G, int M, int K, int N,
                                      bool block512, bool acc_bf16, bool rhs_first, uint16_t* out, int* status,
                                      hipStream_t stream);

// bf16 measurement arm of the forward: the FP8 forward's kernel on bf16 operands.
hipError_t launch_gmm_bf16_fwd(const uint16_t* lhs, const uint16_t* w, const int* group_sizes, int G, int M, int K,
                               int N, bool swiglu, uint16_t* out, int* status, hipStream_t stream);

// tgmm: workspace holds the transposed decoded operands and the scales.
size_t tgmm_workspace_bytes(long long M, long long K, long long N, int G);
hipError_t launch_tgmm_quant(const uint16_t* lhs, const uint16_t* dout, const int* group_sizes, int G, int M, int K,
                             int N, bool grad_e5m2, float* drhs, float* dbg_sl, float* dbg_sd, void* ws,
                             int* status, hipStream_t stream);

// Buffer-wide baseline of the tgmm's operand quantization (every row of the buffer).
size_t tgmm_dense_workspace_bytes(long long M, long long K, long long N, int G);
hipError_t launch_tgmm_dense(const uint16_t* lhs, const uint16_t* dout, const int* group_sizes, int G, int M, int K,
                             int N, bool grad_e5m2, float* drhs, float* dbg_srow, float* dbg_scol, void* ws,
                             int* status, hipStream_t stream);
hipError_t launch_quant_rows_e4m3_all(const uint16_t* lhs, int M, int K, uint8_t* codes, float* scales,
                                      hipStream_t stream);

hipError_t launch_dequant(const uint8_t* codes, const float* scale, int G, long long K, long long N, uint16_t* out,
                          hipStream_t stream);

}  // namespace fp8gmm

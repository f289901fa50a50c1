/*
 * fp8_moe_grouped.h -- C ABI of the MI355X (gfx950) routed-expert FP8 grouped
 * matmul library (libfp8_moe_grouped.so).
 *
 * The operations restate two pages:
 *   "MoE: native FP8 QAT for routed-expert GMMs" (maxtext PR #5969), with its
 *   conversation page, and "MoE fp8 backward: in-kernel drhs operand
 *   quantization + configurable gradient dtype" (maxtext PR #4971).
 * Each declaration names the page and the section it follows.
 *
 * Common conventions
 * ------------------
 * - Every pointer argument except `stream`, `dev_status` and the debug outputs
 *   is a device pointer to caller-owned memory.  The library never allocates,
 *   frees or synchronises; each call only enqueues kernels on `stream`
 *   (a hipStream_t; NULL is the null stream) and returns.
 * - Tensors are row-major and contiguous with 16-byte aligned base pointers.
 *   bf16 tensors are passed as `void*` holding IEEE bfloat16 bit patterns.
 *   Inputs are never written and must not alias outputs or the workspace.
 * - The static ragged buffer: lhs/dout have M rows.  Rows
 *   [off_g, off_g + group_sizes[g]) belong to expert g, off_g = sum of the
 *   sizes before g ("MoE fp8 backward: in-kernel drhs operand quantization + configurable gradient dtype", What: only the tiles covered by group_sizes are
 *   touched).  Rows at or past sum(group_sizes) are stale: never read and,
 *   in row outputs, never written.  `group_sizes` is an int32[G] device array;
 *   a negative size counts as 0 and the running sum is clamped to M, so no
 *   access leaves the buffer.  Such repairs OR bits into *dev_status (device
 *   int32, may be NULL): FP8GMM_DEV_SUM_CLAMPED, FP8GMM_DEV_NEGATIVE_SIZE.
 * - Weight codes are e4m3fn bytes [G, K, N] (N fastest) with one f32 scale
 *   per (expert, output channel), scale[G, N] ("MoE: native FP8 QAT for routed-expert GMMs" Data flow table).
 * - Pointers to buffers with M rows may be NULL when M == 0.
 * - Host-checkable errors return before any HIP call; a failed launch returns
 *   FP8GMM_ERR_HIP.  Outputs are then unspecified.
 * - Shape limits: 0 <= M < 2^24, 1 <= G <= 1024, K and N multiples of 128,
 *   K * N < 2^31, K <= 16384 for ops that quantize activation rows.
 */
#ifndef FP8_MOE_GROUPED_H
#define FP8_MOE_GROUPED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return status */
#define FP8GMM_OK 0
#define FP8GMM_ERR_NULL (-1)        /* a required pointer is NULL */
#define FP8GMM_ERR_SHAPE (-2)       /* a size is out of range */
#define FP8GMM_ERR_UNSUPPORTED (-3) /* a valid request this build does not implement */
#define FP8GMM_ERR_ALIGN (-4)       /* a base pointer is not 16-byte aligned */
#define FP8GMM_ERR_WORKSPACE (-5)   /* workspace NULL or smaller than fp8gmm_workspace_bytes */
#define FP8GMM_ERR_HIP (-6)         /* a kernel launch failed */
#define FP8GMM_ERR_SCRATCH (-7)     /* input larger than gmm_fp8_fwd_noalloc's fixed scratch */

/* bits of *dev_status */
#define FP8GMM_DEV_SUM_CLAMPED 1    /* sum(group_sizes) > M, clamped */
#define FP8GMM_DEV_NEGATIVE_SIZE 2  /* a negative size was treated as 0 */

/* 8-bit formats of the tgmm gradient operand */
#define FP8GMM_E4M3 0
#define FP8GMM_E5M2 1

/* op ids of fp8gmm_workspace_bytes */
#define FP8GMM_OP_FWD 0
#define FP8GMM_OP_SILU 1
#define FP8GMM_OP_DLHS 2
#define FP8GMM_OP_TGMM 3
#define FP8GMM_OP_BF16_FWD 4
#define FP8GMM_OP_BF16_DLHS 5
#define FP8GMM_OP_FFN_FWD 6   /* moe_ffn_fp8_fwd: pass K = H, N = I */
#define FP8GMM_OP_FFN_BWD 7   /* moe_ffn_fp8_bwd: pass K = H, N = I, tile_m = 512 */
#define FP8GMM_OP_FWD_VARIANT 8 /* gmm_fp8_fwd_variant: pass lhs_block as tile_m */
#define FP8GMM_OP_TGMM_DENSE 9  /* tgmm_dense_quant */

/* flags of gmm_fp8_fwd_variant */
#define FP8GMM_LHS_SCALE_BF16 1   /* round each activation scale to bf16 */
#define FP8GMM_ACC_BF16 2         /* bf16 accumulator across the 512-column blocks */
#define FP8GMM_RHS_SCALE_FIRST 4  /* multiply by the weight scale before the activation scale */

/*
 * gmm_fp8_fwd -- native FP8 forward GMM ("MoE: native FP8 QAT for routed-expert GMMs" Description: the forward GMMs
 * run FP8 x FP8, read the codes and per-channel scale directly and quantize
 * the activation inside the op; Implementation: one f32 scale per row over
 * the full K, max(amax, 1e-12)/448, f32 accumulation).
 *
 *   s[r]    = f32( max(max_k |lhs[r,k]|, 1e-12) / 448 )
 *   q[r,k]  = e4m3fn( f32(lhs[r,k] / s[r]) )   saturating, round to nearest even
 *   out[r,n]= bf16( (sum_k q[r,k] * codes[g,k,n]) * s[r] * scale[g,n] )
 *
 * lhs        bf16 [M, K]
 * codes      u8   [G, K, N]     e4m3fn weight codes
 * scale      f32  [G, N]
 * group_sizes i32 [G]
 * out        bf16 [M, N]        rows >= sum(group_sizes) are not written
 * dbg_codes  u8   [M, K] or NULL: receives q (the codes the GEMM consumes)
 * dbg_scale  f32  [M] or NULL:    receives s
 * ws         device workspace of ws_bytes >= fp8gmm_workspace_bytes(FP8GMM_OP_FWD, ...)
 */
int gmm_fp8_fwd(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                int64_t M, int64_t K, int64_t N, int32_t G, void* out, uint8_t* dbg_codes, float* dbg_scale,
                void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/*
 * gmm_fp8_fwd_noalloc -- gmm_fp8_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results, with no workspace and no
 * debug outputs.  The activation codes and row scales go to a fixed scratch
 * array inside the library, FP8GMM_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the library's load until the process ends.  The call allocates and frees
 * nothing.  It needs A256(M*K) + A256(4*M) <= FP8GMM_NOALLOC_SCRATCH_BYTES
 * (A256: rounded up to a multiple of 256), else it returns FP8GMM_ERR_SCRATCH
 * before any HIP call (e.g. up to 4096 rows at K = 7168).  The current
 * device's scratch is used, so `stream` must belong to the current device.
 * All calls on one GPU share that GPU's scratch: calls that may overlap on
 * one GPU (other streams, other threads) race and must be serialised by the
 * caller.  Nothing in the scratch needs clearing between calls (every value
 * read is written earlier in the same call).  Other arguments and errors as
 * gmm_fp8_fwd.
 */
#define FP8GMM_NOALLOC_SCRATCH_BYTES (32u << 20)
int gmm_fp8_fwd_noalloc(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                        int64_t M, int64_t K, int64_t N, int32_t G, void* out, int32_t* dev_status, void* stream);

/*
 * gmm_silu_fp8 -- gmm_fp8_fwd with a fused SwiGLU epilogue for wi ("MoE: native FP8 QAT for routed-expert GMMs"
 * Implementation: gmm_silu_fp8).  The N = 2*I weight columns are [gate | up];
 * with y the scaled f32 GEMM result of gmm_fp8_fwd (before rounding):
 *   out[r,i] = bf16( silu(y[r,i]) * y[r,I+i] ),  silu(z) = z / (1 + exp(-z))
 * out is bf16 [M, I].  I must be a multiple of 128.
 * preact bf16 [M, N] or NULL: receives the pre-activation bf16(y) (exactly
 *   what gmm_fp8_fwd returns for the same inputs), the residual the fused
 *   dSwiGLU backward (gmm_dswiglu_fp8) reads.  Other arguments as above.
 */
int gmm_silu_fp8(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                 int64_t M, int64_t K, int64_t N, int32_t G, void* out, void* preact, uint8_t* dbg_codes,
                 float* dbg_scale, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/*
 * The forward in two calls, for callers whose activations are already e4m3
 * codes with one f32 scale per row (for example after an FP8 all-gather of
 * tokens), or that time the two kernels separately.  gmm_fp8_fwd is exactly
 * quantize_rows_fp8 followed by gmm_fp8_fwd_q (gmm_silu_fp8: gmm_silu_fp8_q).
 *
 * quantize_rows_fp8: for the valid rows r (r < sum(group_sizes), clamped),
 *   scale_out[r] = s[r] and codes_out[r,:] = q[r,:] as defined for
 *   gmm_fp8_fwd; other rows are not written.  lhs bf16 [M, K],
 *   codes_out u8 [M, K], scale_out f32 [M].
 * gmm_fp8_fwd_q / gmm_silu_fp8_q: the GEMM and epilogue of gmm_fp8_fwd /
 *   gmm_silu_fp8 on activation codes aq u8 [M, K] and row scales ascale
 *   f32 [M] (only valid rows are read).  No workspace.
 */
int quantize_rows_fp8(const void* lhs, const int32_t* group_sizes, int64_t M, int64_t K, int32_t G,
                      uint8_t* codes_out, float* scale_out, void* stream);
int gmm_fp8_fwd_q(const uint8_t* aq, const float* ascale, const uint8_t* codes, const float* scale,
                  const int32_t* group_sizes, int64_t M, int64_t K, int64_t N, int32_t G, void* out,
                  int32_t* dev_status, void* stream);
int gmm_silu_fp8_q(const uint8_t* aq, const float* ascale, const uint8_t* codes, const float* scale,
                   const int32_t* group_sizes, int64_t M, int64_t K, int64_t N, int32_t G, void* out, void* preact,
                   int32_t* dev_status, void* stream);

/*
 * gmm_fp8_fwd_variant -- the forward with the LHS-quantization options kept for
 * benchmarks and tests ("MoE: native FP8 QAT for routed-expert GMMs" Implementation: lhs_quant_block_size 512 or the
 * full K, lhs_f32_scale, rhs_scale_first; the bf16 scale per 512 columns with a
 * bf16 accumulator was the earlier default).  lhs_block 0 = one scale per row
 * over the full K, 512 = one scale per 512 columns (the last block may be
 * shorter).  For block b of row r with P_b[r,n] = sum_{k in b} q[r,k] * codes[g,k,n]:
 *   s_b      = f32( max(amax_b, 1e-12) / 448 ), then bf16(s_b) with FP8GMM_LHS_SCALE_BF16
 *   q[r,k]   = e4m3fn( f32(lhs[r,k] / s_b) )
 *   t_b[r,n] = (P_b * s_b) * scale[g,n]   ((P_b * scale[g,n]) * s_b with FP8GMM_RHS_SCALE_FIRST), f32
 *   out      = bf16( sum_b t_b ), or with FP8GMM_ACC_BF16 (lhs_block 512 only) a <- bf16(a + t_b) in
 *              block order and out = a
 * lhs_block 0 with flags 0 is gmm_fp8_fwd bit for bit.  N must be a multiple of 128;
 * no SwiGLU.  dbg_scale (or NULL) receives the scales, f32 [M, nb] with nb =
 * ceil(K/512) or 1.  ws: fp8gmm_workspace_bytes(FP8GMM_OP_FWD_VARIANT, M, K, N, G, lhs_block).
 */
int gmm_fp8_fwd_variant(const void* lhs, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                        int64_t M, int64_t K, int64_t N, int32_t G, int32_t lhs_block, int32_t flags, void* out,
                        uint8_t* dbg_codes, float* dbg_scale, void* ws, size_t ws_bytes, int32_t* dev_status,
                        void* stream);

/*
 * gmm_dlhs_fp8 -- backward dLHS reading the FP8 codes ("MoE: native FP8 QAT for routed-expert GMMs" Description: the
 * dLHS GMM reads the codes and dequantizes each tile on chip, no bf16 weight
 * copy is written to HBM, bit-identical to the dequant path; Implementation:
 * rhs_contract_dequant):
 *   w[g,k,n]    = bf16( f32(codes[g,k,n] * scale[g,n]) )   (as dequantize_fp8_codes)
 *   dlhs[r,k]   = bf16( sum_n dout[r,n] * w[g,k,n] )        f32 accumulation
 * dout bf16 [M, N]; dlhs bf16 [M, K] (rows >= sum(group_sizes) not written).
 * When the contraction N is at most 512, each 128-column block of w is
 * decoded once and kept on chip for a chunk of up to 2048 rows of its expert
 * (same Implementation section: with one K tile the dequantized block is
 * cached across its m tiles); otherwise each tile is decoded as it is used.
 * Both give the same bits.  The call needs no workspace (ws may be NULL).
 */
int gmm_dlhs_fp8(const void* dout, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                 int64_t M, int64_t K, int64_t N, int32_t G, void* dlhs, void* ws, size_t ws_bytes,
                 int32_t* dev_status, void* stream);

/*
 * gmm_dswiglu_fp8 -- backward dLHS of the wo GMM fused with the SwiGLU
 * derivative ("MoE: native FP8 QAT for routed-expert GMMs" Implementation: gmm_dswiglu_fp8 is the wo op,
 * _run_wo_gmm_dswiglu; its forward is gmm_fp8_fwd).  With the wo weight
 * codes [G, K, N] (K = I, the SwiGLU width; N = H, the model width), the wo
 * output gradient dout bf16 [M, N] and the wi pre-activation preact bf16
 * [M, 2K] = [gate | up] kept by gmm_silu_fp8:
 *   dh[r,k]          = sum_n dout[r,n] * w[g,k,n]     f32, not rounded (w as in gmm_dlhs_fp8)
 *   sigma            = 1 / (1 + exp(-gate[r,k]))
 *   d_preact[r,k]    = bf16( dh * up[r,k] * sigma * (1 + gate * (1 - sigma)) )
 *   d_preact[r,K+k]  = bf16( dh * gate * sigma )
 * d_preact bf16 [M, 2K] is the gradient of the wi pre-activation (rows >=
 * sum(group_sizes) not written); it feeds gmm_dlhs_fp8 with the wi codes and
 * tgmm_quant for the wi weight gradient.  Other arguments as gmm_dlhs_fp8.
 */
int gmm_dswiglu_fp8(const void* dout, const uint8_t* codes, const float* scale, const int32_t* group_sizes,
                    const void* preact, int64_t M, int64_t K, int64_t N, int32_t G, void* d_preact,
                    int32_t* dev_status, void* stream);

/*
 * tgmm_quant -- weight gradient with in-kernel operand quantization ("MoE fp8 backward: in-kernel drhs operand quantization + configurable gradient dtype"
 * What: moe_bwd_inkernel_quant quantizes the drhs operands per gm-tile and per
 * channel, touching only rows covered by group_sizes; bwd_quantization_dtype
 * selects e5m2 or e4m3 for the gradient).
 * For each expert g and each buffer-aligned tile t (rows [t*tile_m,
 * (t+1)*tile_m)) with T = rows(g) intersect tile non-empty:
 *   sL[k] = f32(max(max_{r in T} |lhs[r,k]|, 1e-12) / 448)
 *   sD[n] = f32(max(max_{r in T} |dout[r,n]|, 1e-12) / FMAX)   FMAX = 448 (e4m3) or 57344 (e5m2)
 *   drhs[g,k,n] = f32( sum_t sL[k] sD[n] sum_{r in T} e4m3(lhs[r,k]/sL[k]) * grad(dout[r,n]/sD[n]) )
 * Experts without rows get exact zeros.  drhs f32 [G, K, N] is written fully.
 * lhs bf16 [M, K]; dout bf16 [M, N]; grad_dtype FP8GMM_E4M3 or FP8GMM_E5M2;
 * tile_m must be 512 (K and N multiples of 128, as everywhere).  dbg_sL f32 [Tn, K] / dbg_sD f32 [Tn, N] (or NULL)
 * receive the scales of the Tn non-empty (expert, tile) pairs in (expert,
 * tile) order; Tn <= ceil(M/tile_m) + G - 1.
 * ws: fp8gmm_workspace_bytes(FP8GMM_OP_TGMM, M, K, N, G, 512) bytes.  After
 * the call it holds the quantized operands, readable for checks: with
 * Tmax = ceil(M/512) + G - 1 and A(x) = x rounded up to a multiple of 256,
 * qL u8 [Tmax][512][K] at byte 0 and qD u8 [Tmax][512][N] at byte
 * A(Tmax*512*K); slab p (p < Tn) holds pair p's rows in order, then zero
 * codes up to the next multiple of 32 rows (later rows are not written).
 * Next come the pairs' scales (f32 [Tmax][K] at A(Tmax*512*K) + A(Tmax*512*N),
 * f32 [Tmax][N] after it, A-aligned) and, at byte A(Tmax*512*K) +
 * A(Tmax*512*N) + A(Tmax*K*4) + A(Tmax*N*4), the GEMM's work-item deal:
 * int32 [G] block offsets, expert g's work item j (an output tile) going to
 * GEMM block (offset[g] + j) mod the GEMM's grid.  The deal only balances the
 * blocks' work; it is written when G <= 256 (else the deal is round-robin).
 */
int tgmm_quant(const void* lhs, const void* dout, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
               int32_t G, int32_t grad_dtype, int32_t tile_m, float* drhs, float* dbg_sL, float* dbg_sD, void* ws,
               size_t ws_bytes, int32_t* dev_status, void* stream);

/*
 * tgmm_dense_quant -- the buffer-wide backward quantization that tgmm_quant
 * replaces, kept as a measurement baseline ("MoE fp8 backward: in-kernel drhs
 * operand quantization + configurable gradient dtype", What: before the
 * in-kernel path, the lhs rows were quantized again with one scale each, that
 * scale was folded into the gradient and the gradient got one scale per
 * column, all over the static buffer; an Inf in a stale row then reaches a
 * column scale and the weight gradient becomes NaN).  Over EVERY
 * row r < M of the buffer, stale rows included (amax ignores NaN):
 *   sL[r]   = f32(max(max_k |lhs[r,k]|, 1e-12) / 448),   qL = e4m3(f32(lhs / sL))
 *   d'[r,n] = f32(dout[r,n] * sL[r])
 *   sD[n]   = f32(max(max_r |d'[r,n]|, 1e-12) / FMAX),   qD = grad(f32(d' / sD))
 *   drhs[g,k,n] = f32( sD[n] * sum_{r in rows(g)} qL[r,k] * qD[r,n] )
 * so an Inf in any stale row makes every non-empty expert's gradient NaN;
 * experts without rows get zeros.  Arguments as tgmm_quant (no tile_m);
 * dbg_row_scale f32 [M] / dbg_col_scale f32 [N] (or NULL) receive sL / sD.
 * ws: fp8gmm_workspace_bytes(FP8GMM_OP_TGMM_DENSE, M, K, N, G, 0) bytes.
 */
int tgmm_dense_quant(const void* lhs, const void* dout, const int32_t* group_sizes, int64_t M, int64_t K,
                     int64_t N, int32_t G, int32_t grad_dtype, float* drhs, float* dbg_row_scale,
                     float* dbg_col_scale, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);

/*
 * dequantize_fp8_codes -- out[g,k,n] = bf16( f32(codes[g,k,n] * scale[g,n]) )
 * ("MoE: native FP8 QAT for routed-expert GMMs" Implementation: dequantize_fp8_codes).  codes u8 [G, K, N],
 * scale f32 [G, N], out bf16 [G, K, N].  N must be a multiple of 16.
 */
int dequantize_fp8_codes(const uint8_t* codes, const float* scale, int32_t G, int64_t K, int64_t N, void* out,
                         void* stream);

/*
 * bf16 measurement arm: the same group schedule, copy ring, wave layout and
 * epilogues as the FP8 kernels with bf16 weights w[G, K, N] (for example the
 * output of dequantize_fp8_codes) and no activation quantization.  It is the
 * bf16 GMM the FP8 forward is compared against ("MoE: native FP8 QAT for routed-expert GMMs" Tests: kernel
 * microbenchmark, the bf16 arm gets a weight dequantized beforehand), and
 * gmm_bf16_dlhs(dout, dequantize_fp8_codes(codes, scale)) is bit-identical to
 * gmm_dlhs_fp8(dout, codes, scale).
 *   gmm_bf16_fwd : out[r,n]  = bf16( sum_k lhs[r,k] * w[g,k,n] ),  out bf16 [M, N]
 *   gmm_bf16_silu: with y[r,n] = sum_k lhs[r,k] * w[g,k,n] (f32) over N = 2*I
 *                  columns [gate | up], out[r,i] = bf16( silu(y[r,i]) * y[r,I+i] ), out bf16 [M, I]
 *   gmm_bf16_dlhs: dlhs[r,k] = bf16( sum_n dout[r,n] * w[g,k,n] ), dlhs bf16 [M, K]
 * K * N * 2 must be below 2^32 for the forward arms.
 */
int gmm_bf16_fwd(const void* lhs, const void* w, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
                 int32_t G, void* out, int32_t* dev_status, void* stream);
int gmm_bf16_silu(const void* lhs, const void* w, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
                  int32_t G, void* out, int32_t* dev_status, void* stream);
int gmm_bf16_dlhs(const void* dout, const void* w, const int32_t* group_sizes, int64_t M, int64_t K, int64_t N,
                  int32_t G, void* dlhs, int32_t* dev_status, void* stream);

/*
 * One routed-expert FFN on a static ragged buffer, forward and backward, as
 * the calls above chain them ("MoE: native FP8 QAT for routed-expert GMMs" Implementation: gmm_up_or_silu runs
 * gmm_silu_fp8 for wi and _run_wo_gmm_dswiglu runs gmm_dswiglu_fp8 for wo;
 * "MoE fp8 backward: in-kernel drhs operand quantization + configurable gradient dtype" What: both weight gradients are tgmm_quant).  x bf16 [M, H];
 * wi codes [G, H, 2I] with scale [G, 2I]; wo codes [G, I, H] with scale
 * [G, H].  H and I must be multiples of 256 and at most 16384.
 *
 * moe_ffn_fp8_fwd: h = gmm_silu_fp8(x, wi) bf16 [M, I] with preact bf16
 *   [M, 2I] (may be NULL when no backward follows), then
 *   y = gmm_fp8_fwd(h, wo) bf16 [M, H].  ws: fp8gmm_workspace_bytes(
 *   FP8GMM_OP_FFN_FWD, M, H, I, G, 0) bytes.
 * moe_ffn_fp8_bwd: from the forward's x, h, preact and the output gradient
 *   dy bf16 [M, H]:
 *     d_preact = gmm_dswiglu_fp8(dy, wo, preact)          bf16 [M, 2I]
 *     dx       = gmm_dlhs_fp8(d_preact, wi)               bf16 [M, H]  (dx may be NULL: skipped)
 *     dwo      = tgmm_quant(h, dy, grad_dtype)            f32 [G, I, H]
 *     dwi      = tgmm_quant(x, d_preact, grad_dtype)      f32 [G, H, 2I]
 *   tile_m is 512.  ws: fp8gmm_workspace_bytes(FP8GMM_OP_FFN_BWD, M, H, I, G, 512).
 * Both enqueue their kernels in that order on `stream`; results are those of
 * the individual calls, bit for bit.
 */
int moe_ffn_fp8_fwd(const void* x, const uint8_t* wi_codes, const float* wi_scale, const uint8_t* wo_codes,
                    const float* wo_scale, const int32_t* group_sizes, int64_t M, int64_t H, int64_t I, int32_t G,
                    void* h, void* preact, void* y, void* ws, size_t ws_bytes, int32_t* dev_status, void* stream);
int moe_ffn_fp8_bwd(const void* x, const void* h, const void* preact, const void* dy, const uint8_t* wi_codes,
                    const float* wi_scale, const uint8_t* wo_codes, const float* wo_scale,
                    const int32_t* group_sizes, int64_t M, int64_t H, int64_t I, int32_t G, int32_t grad_dtype,
                    void* d_preact, void* dx, float* dwi, float* dwo, void* ws, size_t ws_bytes,
                    int32_t* dev_status, void* stream);

/*
 * fp8gmm_workspace_bytes -- device workspace the call `op` needs for these
 * sizes (0 if none).  Returns 0 as well for sizes the op rejects.
 */
size_t fp8gmm_workspace_bytes(int32_t op, int64_t M, int64_t K, int64_t N, int32_t G, int32_t tile_m);

/* fp8gmm_status_string -- static text of a status code. */
const char* fp8gmm_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* FP8_MOE_GROUPED_H */

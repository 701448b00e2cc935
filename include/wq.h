/*
 * wq.h -- C ABI of the MI355X (gfx950) block-scaled quantizers and the
 * weight-only quantized matmul y = x . dequant(Wq)^T.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named x, codes, scales, wq, y, ... are DEVICE pointers owned by
 *   the caller (typically PyTorch tensors).  The library never allocates,
 *   frees or synchronises; all work is enqueued asynchronously on `stream`
 *   (a hipStream_t; NULL means the default stream).
 * - Every buffer is dense and row-major ("contiguous"); the row stride is the
 *   row length.  Base pointers must be 16-byte aligned (WQ_EALIGN otherwise).
 * - Shapes and divisibility are validated on the host before anything is
 *   launched: violations return WQ_EINVAL, unsupported dtype/block/group
 *   combinations WQ_EUNSUPPORTED, launch failures WQ_EHIP.  An error return
 *   means nothing was enqueued.
 * - Out-of-range values never raise: they saturate, as the formats define.
 * - Element counts are int64_t; rows * cols must fit in 2^40.
 *
 * Formats
 * -------
 * WQ_E4M3    OCP FP8 E4M3 "fn": 1 byte, bias 7, no inf, 0x7F/0xFF NaN, max 448.
 * WQ_E2M1X2  FP4 E2M1, two codes per byte, element 2j in the low nibble of byte j.
 * WQ_E8M0    unsigned power-of-two scale, 1 byte, value 2^(c-127).
 * WQ_INT4X8  signed INT4 (two's complement), eight per uint32, element 8i+j in
 *            bits 4j..4j+3 of word i.
 * WQ_BF16    bfloat16 bit patterns (uint16).
 * WQ_F32     IEEE binary32.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WQ_OK = 0,
  WQ_EINVAL = 1,        /* bad shape, size, NULL pointer or divisibility     */
  WQ_EALIGN = 2,        /* a base pointer is not 16-byte aligned              */
  WQ_EUNSUPPORTED = 3,  /* dtype / block / group combination not implemented  */
  WQ_EHIP = 4           /* a HIP launch or runtime call failed               */
} wq_status;

typedef enum {
  WQ_F32 = 0,
  WQ_BF16 = 1,
  WQ_E4M3 = 2,
  WQ_E2M1X2 = 3,
  WQ_E8M0 = 4,
  WQ_INT4X8 = 5
} wq_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* wq_status_string(int status);

/*
 * quantize_e4m3 -- fp32/bf16 -> FP8 E4M3, round to nearest even, saturating.
 *
 * Defined by FreeToken PR #805 (a single round-to-nearest-even conversion from
 * fp32 with saturation to +-448: 200.04 -> 208) and by "Numerics: FP32 to INT4,
 * and why bf16 won", fp8 linear walkthrough steps 1-2 (dynamic scale = amax /
 * 448 in fp32; the values divided by the scale in fp32; saturating clamp;
 * narrowing cast).
 *
 * x       rows x cols, dtype x_dtype (WQ_F32 or WQ_BF16).
 * block   0   plain cast, no scale (`scales` may be NULL);
 *         >0  one fp32 scale per 1 x block group along a row, block in
 *             {16, 32, 64, 128, 256}; cols % block == 0;
 *         -1  one fp32 scale per row.
 * codes   rows x cols bytes (output).
 * scales  rows x (cols/block) fp32, or rows x 1 for block == -1 (output).
 * Scale = RN_f32(amax / 448), replaced by 1.0 when it is zero.  Codes are
 * e4m3(RN_f32(x / scale)) with correctly rounded fp32 division.  NaN input to
 * the plain cast gives 0x7F with the input's sign; +-inf gives +-448.  For the
 * scaled modes a group holding a non-finite value is outside the contract: the
 * call succeeds but that group's codes and scale are unspecified.
 * cols % 8 == 0 is required in every mode.
 */
wq_status quantize_e4m3(const void* x, int x_dtype, int64_t rows, int64_t cols,
                        int32_t block, uint8_t* codes, float* scales, void* stream);

/*
 * quantize_mxfp4 -- fp32/bf16 -> MXFP4 (E2M1 element codes + E8M0 block scale).
 *
 * Defined by "Fix the E8M0 scale computation in the MXFP4 (W4A4) MOE CUTLASS
 * kernel" (vLLM PR #43557), section "Fix: Exponent-First with 0.75-Threshold
 * Rounding": per block, bits = fp32 pattern of max|x|; the biased exponent of
 * (bits + 2^21) & 0xFF800000, minus 2 and clamped at 0, is the E8M0 code c.
 * Elements are x * 2^(127-c) rounded to the nearest E2M1 value (ties to even
 * code), saturating at 6 ("Numerics: FP32 to INT4, and why bf16 won", section
 * "MXFP4 and the block-scaled family").
 *
 * x       rows x cols, dtype x_dtype (WQ_F32 or WQ_BF16); block in {16, 32};
 *         cols % 32 == 0.
 * codes   rows x cols/2 bytes (output), element 2j in the low nibble of byte j.
 * scales  rows x cols/block E8M0 bytes (output).
 * Blocks holding a non-finite value are outside the contract (unspecified
 * codes and scale, no error).
 */
wq_status quantize_mxfp4(const void* x, int x_dtype, int64_t rows, int64_t cols,
                         int32_t block, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * quantize_int4 -- fp32/bf16 weights -> symmetric INT4 with bf16 group scales.
 *
 * Follows "Numerics: FP32 to INT4, and why bf16 won" (x = s * (q - z), z = 0;
 * s = max|x| / qmax; an all-zero group gets s = 1; int4 range [-8, 7]; one
 * 16-bit scale per 128-element group along K).  s = bf16(RN_f32(amax / 7))
 * (replaced by 1.0 if zero); q = clamp(rint(RN_f32(x / s)), -8, 7).
 *
 * w       rows x cols (N x K), dtype w_dtype (WQ_F32 or WQ_BF16).
 * group   32, 64 or 128; cols % group == 0 and cols % 32 == 0.
 * packed  rows x cols/8 uint32 (output, WQ_INT4X8 layout).
 * scales  rows x cols/group bf16 bit patterns (output).
 * Groups holding a non-finite value are outside the contract.
 */
wq_status quantize_int4(const void* w, int w_dtype, int64_t rows, int64_t cols,
                        int32_t group, uint32_t* packed, uint16_t* scales, void* stream);

/*
 * wq_dequant -- packed weights + scales -> the bf16 operand the matmul uses.
 *
 * "Your 3090 Isn't Missing Anything for FP8/NVFP4 Weight-Only Inference",
 * section "4.1 The Marlin implementation": weights are converted to bf16 in
 * registers; every E4M3 and E2M1 value is exact in bf16.
 *   w_dtype WQ_INT4X8 + s_dtype WQ_BF16  (group 32/64/128): bf16(q * s), one
 *       rounding of the exact product.
 *   w_dtype WQ_E2M1X2 + s_dtype WQ_E8M0  (group 16/32): bf16(v * 2^(c-127)),
 *       exact; scale code 255 (E8M0 NaN) is outside the contract.
 *   w_dtype WQ_E4M3  (s_dtype WQ_F32, scales may be NULL; group ignored):
 *       bf16(v), exact; the per-channel scale is NOT applied (it multiplies the
 *       fp32 accumulator).  NaN codes give a NaN of unspecified sign.
 * wq      N x K elements in the w_dtype layout; w_scales N x K/group.
 * w_bf16  N x K bf16 (output).  K % 32 == 0.
 */
wq_status wq_dequant(const void* wq, int w_dtype, const void* w_scales, int s_dtype,
                     int32_t group, int64_t N, int64_t K, uint16_t* w_bf16, void* stream);

/*
 * wq_gemm -- y[M,N] = x[M,K] . dequant(Wq[N,K])^T, bf16 x, fp32 accumulation,
 * bf16 y (one rounding at the end).
 *
 * "Numerics: FP32 to INT4, and why bf16 won" (narrow storage, fp32 accumulate,
 * one narrowing cast; per-channel scales factor out of the dot product, group
 * scales fold inside the K loop) and "Your 3090 Isn't Missing Anything...",
 * sections 2 and 4.1 (bf16 x bf16 multiply after in-register dequantization).
 *
 * Weight/scale pairs:
 *   WQ_INT4X8 + WQ_BF16  group in {32, 64, 128}
 *   WQ_E2M1X2 + WQ_E8M0  group 32
 *   WQ_E4M3   + WQ_F32   group == K (one fp32 scale per output channel, applied
 *                         to the fp32 accumulator before the bf16 rounding)
 * M >= 1, N >= 1, K % 128 == 0.  M <= 16 runs the split-K decode kernel,
 * larger M the MFMA prefill kernel.
 * workspace / ws_bytes: reserved; the current kernels need none
 * (wq_gemm_workspace_size returns 0) and accept NULL / 0.
 * Accuracy contract: |y - y_ref| <= 8e-3 |y_ref| + 1e-3 sum_k |x_k w_k| per
 * element, y_ref the exact product of the dequantized operands.
 */
wq_status wq_gemm(const void* x_bf16, int64_t M, int64_t N, int64_t K,
                  const void* wq, int w_dtype, const void* w_scales, int s_dtype,
                  int32_t group, void* y_bf16, void* workspace, size_t ws_bytes,
                  void* stream);

/* Bytes of workspace wq_gemm needs for this problem (currently always 0). */
size_t wq_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int w_dtype, int32_t group);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */

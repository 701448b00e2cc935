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
 * WQ_UINT4X8 unsigned INT4 codes 0..15, eight per uint32 in the WQ_INT4X8
 *            nibble order.
 * WQ_BF16Z   one uint32 per group of an asymmetric INT4 tensor: the bf16
 *            scale in bits 0..15, the zero-point (0..15) in bits 16..23, the
 *            rest zero.
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
  WQ_INT4X8 = 5,
  WQ_UINT4X8 = 6,
  WQ_BF16Z = 7
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

/* E8M0 scale rules of quantize_mx; vmax is the fp32 block maximum magnitude,
 * m the element mantissa width (1 for E2M1, 3 for E4M3), off its top binade (2
 * for E2M1, 8 for E4M3), emax its largest value (6 or 448).                  */
typedef enum {
  WQ_MX_ROUND = 0,      /* biased_exp(bits(vmax) + 2^(22-m)) - off, clamped at 0  */
  WQ_MX_HALF = 1,       /* biased_exp(bits(vmax) + 2^22) - off, clamped at 0      */
  WQ_MX_OCP = 2,        /* biased_exp(vmax) - off, clamped at 0                   */
  WQ_MX_FLOOR_DIV = 3,  /* biased_exp(RN_f32(vmax * RN_f32(1/emax)))             */
  WQ_MX_CEIL_DIV = 4    /* max(ceil(log2(RN_f32(vmax / emax))), -127) + 127       */
} wq_mx_rule;

/*
 * quantize_mx -- fp32/bf16 -> MX block format (E2M1 or E4M3 element codes +
 * E8M0 block scale) under a choice of scale rule.
 *
 * Rules: "Fix the E8M0 scale computation in the MXFP4 (W4A4) MOE CUTLASS
 * kernel" (vLLM PR #43557): WQ_MX_ROUND is the rule of section "Fix:
 * Exponent-First with 0.75-Threshold Rounding", with the increment of section
 * "Origin: Matching the Quantization Toolchain" for an m-bit mantissa (2^21 for
 * E2M1, 2^19 for E4M3); WQ_MX_OCP and WQ_MX_HALF are the strict OCP and
 * 0.5-threshold rows of "Why This Helps Precision (Not Strict OCP MX)";
 * WQ_MX_FLOOR_DIV is the old rule of "Root Cause" (the reciprocal is the
 * correctly rounded fp32 one).  WQ_MX_CEIL_DIV is SGLang's quantizer in
 * "Numerics: FP32 to INT4, and why bf16 won", section "MXFP4 and the
 * block-scaled family" (the quotient rounded up to a power of two, exactly).
 * The element formats are from the OCP MX list on that page (mxfp4,
 * mxfp8_e4m3).  An all-zero block gets code 0 under every rule.
 *
 * Elements: v = x * 2^(127-c); E2M1: nearest E2M1 value, ties to even code,
 * saturating at 6 (as quantize_mxfp4); E4M3: RNE, saturating at 448.
 * WQ_MX_ROUND with WQ_E2M1X2 gives exactly the output of quantize_mxfp4.
 *
 * x       rows x cols, dtype x_dtype (WQ_F32 or WQ_BF16); cols % 32 == 0.
 * block   16 or 32.
 * elem    WQ_E2M1X2 (codes rows x cols/2 bytes, element 2j in the low nibble
 *         of byte j) or WQ_E4M3 (codes rows x cols bytes).
 * rule    a wq_mx_rule; anything else is WQ_EINVAL.
 * scales  rows x cols/block E8M0 bytes (output).
 * Blocks holding a non-finite value are outside the contract (unspecified
 * codes and scale, no error).
 */
wq_status quantize_mx(const void* x, int x_dtype, int64_t rows, int64_t cols, int32_t block,
                      int32_t elem, int32_t rule, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * quantize_nvfp4 -- fp32/bf16 -> NVFP4 (E2M1 codes, one E4M3 scale per 16).
 *
 * "Numerics: FP32 to INT4, and why bf16 won", section "MXFP4 and the
 * block-scaled family" (NVFP4: blocks of 16, the scale stored as E4M3, so it
 * has mantissa bits and can sit between powers of two); "Your 3090 Isn't
 * Missing Anything for FP8/NVFP4 Weight-Only Inference", section 2.1 (the
 * block and its E4M3 scale decode to bf16 for a bf16 multiply); and the review
 * note on vLLM PR #43557 (divide the elements by the dequantized scale).
 * Per 1 x 16 block, with g = tensor_scale:
 *   s8 = e4m3(RN_f32(RN_f32(amax / 6) / g)), RNE, saturating at 448;
 *   d = RN_f32(e4m3_value(s8) * g);
 *   code = e2m1(RN_f32(x / d)) (nearest, ties to even code, saturating at 6),
 *   a zero of x's sign when d == 0.
 * Dequantized value: g * e4m3_value(s8) * e2m1_value(code).  The per-tensor
 * scale is not given on the pages; g = 1 is their description.
 *
 * x             rows x cols, dtype x_dtype (WQ_F32 or WQ_BF16); cols % 16 == 0.
 * tensor_scale  finite and > 0 (WQ_EINVAL otherwise).
 * codes         rows x cols/2 bytes (output), element 2j in the low nibble of byte j.
 * scales        rows x cols/16 E4M3 bytes (output).
 * Blocks holding a non-finite value are outside the contract.
 */
wq_status quantize_nvfp4(const void* x, int x_dtype, int64_t rows, int64_t cols,
                         float tensor_scale, uint8_t* codes, uint8_t* scales, void* stream);

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
 * quantize_int4_asym -- fp32/bf16 weights -> asymmetric INT4, x = s * (q - z).
 *
 * "Numerics: FP32 to INT4, and why bf16 won": the affine map with a float
 * scale s and an integer zero-point z (z != 0 covers a range not centred on
 * zero for one extra subtraction in the dequantization, (q - z) * s); the
 * all-zero-group policy s = 1; groups of 32 to 128 along K.  Per group, over a
 * range that contains 0: lo = min(min x, 0), hi = max(max x, 0),
 * s = bf16(RN_f32(RN_f32(hi - lo) / 15)) (1 if zero),
 * z = clamp(rint(RN_f32(-lo / s)), 0, 15), q = clamp(rint(RN_f32(x / s)) + z, 0, 15).
 *
 * w          rows x cols (N x K), dtype w_dtype (WQ_F32 or WQ_BF16).
 * group      32, 64 or 128; cols % group == 0.
 * packed     rows x cols/8 uint32 (output, WQ_UINT4X8).
 * scalezero  rows x cols/group uint32 (output, WQ_BF16Z).
 * Groups holding a non-finite value, or whose range overflows fp32, are
 * outside the contract.
 */
wq_status quantize_int4_asym(const void* w, int w_dtype, int64_t rows, int64_t cols,
                             int32_t group, uint32_t* packed, uint32_t* scalezero, void* stream);

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
 *   w_dtype WQ_UINT4X8 + s_dtype WQ_BF16Z  (group 32/64/128): bf16((q - z) * s),
 *       one rounding of the exact product; s in (0, 2^120], z <= 15.
 *   w_dtype WQ_E2M1X2 + s_dtype WQ_E4M3  (group 16, NVFP4): v * e4m3 value,
 *       exact (every such product is a bf16 number); the per-tensor scale is
 *       not applied (it is wq_gemm's alpha).  NaN scale codes are outside the
 *       contract.
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
 *   WQ_INT4X8 + WQ_BF16  group in {32, 64, 128}; scales in (0, 2^120].  With
 *                         group 128, decode steps whose scales all have 3
 *                         trailing zero mantissa bits (what quantize_int4
 *                         writes) multiply the exact codes and scale the
 *                         group sums; the result is the same product.
 *   WQ_UINT4X8 + WQ_BF16Z  group in {32, 64, 128} (asymmetric INT4, operand
 *                         bf16((q - z) * s)); scales in (0, 2^120], z <= 15
 *   WQ_E2M1X2 + WQ_E8M0  group 32 (MXFP4)
 *   WQ_E2M1X2 + WQ_E4M3  group 16 (NVFP4; the operand is the exact product of
 *                         the E2M1 and E4M3 values)
 *   WQ_E4M3   + WQ_F32   group == K (one fp32 scale per output channel, applied
 *                         to the fp32 accumulator before the bf16 rounding)
 * alpha   an fp32 factor on the accumulator before the bf16 rounding (the
 *         per-tensor scale of NVFP4; 1 otherwise).  Non-finite: WQ_EINVAL.
 *         y = bf16(acc * RN(chan * alpha)) for WQ_E4M3 weights,
 *         y = bf16(acc * alpha) for the others.
 * M >= 1, N >= 1, K % 128 == 0 for every weight format, including INT4
 * groups of 32 or 64 and MXFP4 blocks of 32 (the kernels step K in 128-element
 * chunks of one 16-byte load per lane and have no tail path; a K that is only
 * a multiple of the group returns WQ_EINVAL).  M <= 32 runs the split-K decode kernels;
 * 32 < M <= 64 runs them twice, on rows 0-31 and on the rest (both launches
 * on `stream`); larger M the MFMA prefill kernel, except that for
 * 64 < M <= 256 the decode launches (one per 32 rows) are taken when a cost
 * estimate from M, N, K and the CU count puts them ahead (at small N the
 * prefill kernel's 256 x 256 tiles leave most CUs idle).
 * workspace / ws_bytes: reserved; the current kernels need none
 * (wq_gemm_workspace_size returns 0) and accept NULL / 0.
 * Accuracy contract: |y - y_ref| <= 8e-3 |y_ref| + 1e-3 sum_k |x_k w_k| per
 * element, y_ref the exact product of the dequantized operands.
 */
wq_status wq_gemm(const void* x_bf16, int64_t M, int64_t N, int64_t K,
                  const void* wq, int w_dtype, const void* w_scales, int s_dtype,
                  int32_t group, float alpha, void* y_bf16, void* workspace,
                  size_t ws_bytes, void* stream);

/* Bytes of workspace wq_gemm needs for this problem (currently always 0). */
size_t wq_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int w_dtype, int32_t group);

/*
 * W8A8 FP8 path
 * -------------
 * Defined by "Numerics: FP32 to INT4, and why bf16 won": the Triton
 * block-scaled FP8 GEMM of the section on storage and accumulation dtypes
 * (fp32 accumulator; per K block the fp8 product is scaled by the activation
 * scale of each row and the weight scale of each column; one narrowing cast at
 * the store) and the fp8 linear walkthrough (step 2: divide by the scale in
 * fp32, saturating clamp, conversion; step 3: fp8 x fp8 with both scales
 * folded in inside the K loop, one cast to bf16).  K blocks are 128 wide.
 */

/*
 * quantize_e4m3_static -- per-tensor static E4M3 quantization with a given
 * scale (the per-tensor cast site FreeToken PR #805 lists):
 * codes = e4m3(RN_f32(x / scale)), correctly rounded division, saturating at
 * +-448.
 * x      rows x cols, dtype x_dtype (WQ_F32 or WQ_BF16); cols % 16 == 0.
 * scale  DEVICE pointer to one fp32 value > 0 (read by the kernel, so a
 *        calibrated scale never round-trips through the host).
 * codes  rows x cols bytes (output).
 * Non-finite inputs and non-positive scales are outside the contract.
 */
wq_status quantize_e4m3_static(const void* x, int x_dtype, int64_t rows, int64_t cols,
                               const float* scale, uint8_t* codes, void* stream);

/*
 * quantize_e4m3_block2d -- weights -> E4M3 with one fp32 scale per 128 x 128
 * block: s = RN_f32(amax / 448) (1 if zero), codes e4m3(RN_f32(w / s)).
 * w       rows x cols (N x K), dtype w_dtype (WQ_F32 or WQ_BF16); cols % 128 == 0;
 *         a partial last row block uses the rows it has.
 * codes   rows x cols bytes (output).
 * scales  ceil(rows/128) x cols/128 fp32 (output).
 */
wq_status quantize_e4m3_block2d(const void* w, int w_dtype, int64_t rows, int64_t cols,
                                uint8_t* codes, float* scales, void* stream);

/*
 * wq_gemm_w8a8 -- y[M,N] = sum over K blocks kb of a_s(m,kb) b_s(n,kb) *
 * sum_{k in kb} a[m,k] b[n,k], E4M3 operands, fp32 accumulation, one bf16
 * rounding.
 *
 * a        M x K E4M3 activations.  a_scale: fp32, the scale of (m, kb) is
 *          a_scale[m * as_m + kb * as_k] (per tensor: 0, 0; per token: 1, 0;
 *          per token and 128-wide group: K/128, 1).
 * b        N x K E4M3 weights.  b_scale: fp32, the scale of (n, kb) is
 *          b_scale[(n / group_n) * bs_n + kb * bs_k]; group_n 128 (128 x 128
 *          blocks: bs_n = K/128, bs_k = 1; or one scale per 128 channels) or 1
 *          (per channel, bs_k must be 0); per tensor: bs_n = bs_k = 0.
 * y        M x N bf16 (output).
 * K % 128 == 0.  When a scale depends on kb, every K block's partial sums are
 * scaled before they are added; otherwise the scales multiply the finished
 * fp32 sums.  Scale arrays must hold every index the strides reach; negative
 * strides are WQ_EINVAL.  The fp8 matrix cores treat E4M3 subnormal operands
 * as zero.  Accuracy contract: |y - y_ref| <= 8e-3 |y_ref| + 1e-3 sum_k
 * |a_k s_a b_k s_b|.
 */
wq_status wq_gemm_w8a8(const uint8_t* a, const float* a_scale, int64_t as_m, int64_t as_k,
                       const uint8_t* b, const float* b_scale, int64_t bs_n, int64_t bs_k,
                       int32_t group_n, int64_t M, int64_t N, int64_t K, uint16_t* y,
                       void* stream);

/*
 * W4A8 mixture-of-experts path
 * ----------------------------
 * Defined by "Production-Ready W4A8: vLLM Integration and Quality Recovery
 * Techniques Explained" (Cohere), sections "High-Performance W4A8 GEMM Kernel"
 * (INT4 weights become FP8 through a table of the 16 products s * w of a group's
 * fp8 scale s, built from the scale inside the main loop, then an fp8 x fp8
 * multiply with fp32 accumulation) and "Accurate W4A8 Kernel" (group scales
 * quantized to fp8 with an fp32 channel scale, 1/8 on the fp8 scales and 8 on
 * the channel scale so that every s * w stays in range; per-token and
 * per-channel fp32 scales applied at the end).  INT4 groups are 128 elements
 * along K.
 */

/*
 * wq_moe_route -- softmax over the E expert logits of each token, the k most
 * probable experts, and the grouping of the T*k (token, expert) pairs.
 *
 * logits     T x E fp32.  1 <= k <= E <= 64; T*k < 2^31.
 * ids        T x k int32 (output): experts in decreasing logit order (equal
 *            logits: lower expert id first).
 * weights    T x k fp32 (output): their softmax probabilities (fp32 arithmetic;
 *            not re-normalised).
 * offsets    E + 1 int32 (output): grouped rows of expert e are
 *            [offsets[e], offsets[e + 1]); offsets[E] = T*k.
 * row_token  T*k int32 (output): token of each grouped row, increasing within
 *            an expert.
 * row_slot   T*k int32 (output): position of the expert in that token's ids.
 * Non-finite logits are outside the contract.
 */
wq_status wq_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                       int32_t* offsets, int32_t* row_token, int32_t* row_slot, void* stream);

/*
 * wq_w4a8_prepack -- one-time preparation of INT4 expert weights for
 * wq_moe_gemm_w4a8.
 *
 * wq       experts x N x K/8 uint32 INT4X8 words (group 128 along K).
 * scales   experts x N x K/128 bf16 group scales.
 * wq_out   experts x N x K/8 uint32 (output, may alias wq): the same codes with
 *          the nibbles of every word interleaved (element j < 4 of a word in
 *          nibble 2j, element j >= 4 in nibble 2(j-4)+1), the layout the GEMM's
 *          table lookups read.
 * s8       experts x N x K/128 E4M3 codes (output): e4m3(RN_f32(s / ch)).
 * ch       experts x N fp32 (output): 8 * RN_f32(max_g |s| / 448), with
 *          RN_f32(...) replaced by 1 for an all-zero channel.
 * K % 128 == 0.  Non-finite scales are outside the contract.
 */
wq_status wq_w4a8_prepack(const uint32_t* wq, const uint16_t* scales, int64_t experts, int64_t N, int64_t K,
                          uint32_t* wq_out, uint8_t* s8, float* ch, void* stream);

/*
 * wq_w4a8_dequant -- the E4M3 weights the grouped GEMM multiplies, written
 * out: codes[n, k] = e4m3(w[n, k] * val(s8[n, k / 128])), rounded to nearest
 * even, saturating at 448 (the table lookup of wq_moe_gemm_w4a8, same device
 * code).  wq: N x K/8 words in the wq_w4a8_prepack layout; s8: N x K/128;
 * codes: N x K bytes (output).
 */
wq_status wq_w4a8_dequant(const uint32_t* wq, const uint8_t* s8, int64_t N, int64_t K, uint8_t* codes, void* stream);

/*
 * wq_moe_gemm_w4a8 -- grouped GEMM over experts:
 *   y[r, n] = bf16( a_scale[t] * ch[e, n] * sum_k val(x8[t, k]) * val(W8[e, n, k]) )
 * for grouped row r of expert e (offsets[e] <= r < offsets[e + 1]), token
 * t = row_token[r] (t = r when row_token is NULL, which requires R == T), and
 * W8 the table-looked-up E4M3 weights (see wq_w4a8_dequant), fp32 accumulation.
 *
 * x8        T x K E4M3 codes (per-token quantized activations), a_scale T fp32
 *           (quantize_e4m3 with block -1 produces both).  T*K < 2^31.
 * row_token R int32 or NULL; offsets experts + 1 int32 (device), offsets[0] = 0,
 *           non-decreasing, offsets[experts] = R (wq_moe_route writes such
 *           arrays).  Both are device data the host cannot check; the kernel
 *           clamps every expert's row range to [0, R] (a decreasing or
 *           out-of-range pair of offsets gives an empty expert) and treats a
 *           row_token entry outside [0, T) as a zero row with scale 0, so no
 *           access leaves the buffers, but the rows of such an expert are then
 *           not computed as the formula above states.
 * wq, s8, ch  from wq_w4a8_prepack, experts x N x ...; K % 128 == 0.
 * y         R x N bf16 (output), rows in grouped order.
 * The fp8 MFMA treats E4M3 subnormal operands as zero; results differ from the
 * exact product by at most the flushed terms.
 */
wq_status wq_moe_gemm_w4a8(const uint8_t* x8, int64_t T, const float* a_scale, const int32_t* row_token, int64_t R,
                           const int32_t* offsets, int32_t experts, int64_t N, int64_t K, const uint32_t* wq,
                           const uint8_t* s8, const float* ch, uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */

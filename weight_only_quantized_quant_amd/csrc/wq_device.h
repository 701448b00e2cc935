// Device helpers for the gfx950 quantizer and matmul kernels.
//
// Hardware conversions used here (each checked bit-for-bit against the CPU
// definitions of the formats by the test-suite):
//   v_cvt_pk_bf16_f32            fp32 pair -> bf16 pair, round to nearest even
//   v_cvt_pk_fp8_f32             fp32 pair -> OCP E4M3 pair, RNE; it does NOT
//                                saturate (|x| > 464 gives NaN), so callers clamp
//   v_cvt_scalef32_pk_fp4_f32    fp32 pair -> E2M1 pair of x / 2^(e-127), RNE,
//                                saturating at 6; e = exponent field of `scale`
//   v_cvt_scalef32_pk_bf16_fp4   E2M1 pair -> bf16 pair of v * 2^(e-127), exact
//   v_cvt_scalef32_pk_bf16_fp8   E4M3 pair -> bf16 pair of v * 2^(e-127), exact
// For the scaled forms only the exponent field e of the fp32 scale operand is
// used, i.e. the scale acts as an E8M0 code (e = 0 means 2^-127).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace wq {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair (a in the low half), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float a) { return pack_bf16x2(a, a) & 0xFFFFu; }

// E2M1 pair from byte `sel` of `w` -> bf16 pair scaled by 2^(code-127).
template <int SEL>
__device__ __forceinline__ uint32_t dq_fp4_pair(uint32_t w, float scale_as_e8m0) {
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_as_e8m0, SEL);
  return __builtin_bit_cast(uint32_t, v);
}

// E4M3 pair from half `HI` of `w` -> exact bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t dq_fp8_pair(uint32_t w) {
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, v);
}

// E2M1 word (8 codes) times an fp32 scale s -> 4 bf16 pairs.  The scaled
// conversions read only the exponent of their scale operand, so the codes are
// decoded unscaled (exact fp32), multiplied by s in fp32 and rounded once.  For
// an E4M3-valued s every product is a bf16 number: the result is exact.
template <int SEL>
__device__ __forceinline__ uint32_t dq_fp4_pair_mul(uint32_t w, float s) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return pack_bf16x2(f[0] * s, f[1] * s);
}
__device__ __forceinline__ void dq_nv4_word(uint32_t w, float s, uint32_t out[4]) {
  out[0] = dq_fp4_pair_mul<0>(w, s);
  out[1] = dq_fp4_pair_mul<1>(w, s);
  out[2] = dq_fp4_pair_mul<2>(w, s);
  out[3] = dq_fp4_pair_mul<3>(w, s);
}

// fp32 scale operand whose exponent field is the E8M0 code c (c = 0 -> 0.0f,
// which the scaled conversions read as 2^-127).
__device__ __forceinline__ float e8m0_as_scale(uint32_t c) { return __uint_as_float(c << 23); }

// Exponent-first 0.75-threshold E8M0 rule on the fp32 pattern of max|x|.
__device__ __forceinline__ uint32_t e8m0_code(float vmax) {
  uint32_t bits = __float_as_uint(vmax) & 0x7FFFFFFFu;
  uint32_t be = ((bits + (1u << 21)) & 0xFF800000u) >> 23;
  return be > 2u ? be - 2u : 0u;
}

// Bytes ue (codes of elements 0, 2, 4, 6) and uo (1, 3, 5, 7), each in [0, 15]:
// read as E4M3 codes they are u * 2^-9 exactly (codes 0..7 are the subnormals
// u/8 * 2^-6, codes 8..15 the binade (1 + (u-8)/8) * 2^-6), so one scaled
// conversion with scale 2^9 turns two of them into exact floats.  Then
// fma(u, s, b) and one RNE conversion per pair.
__device__ __forceinline__ void dq_u4_bytes(uint32_t ue, uint32_t uo, float s, float b, uint32_t out[4]) {
  const auto e01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ue, 512.0f, false);
  const auto e23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ue, 512.0f, true);
  const auto o01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(uo, 512.0f, false);
  const auto o23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(uo, 512.0f, true);
  out[0] = pack_bf16x2(__builtin_fmaf(e01[0], s, b), __builtin_fmaf(o01[0], s, b));
  out[1] = pack_bf16x2(__builtin_fmaf(e01[1], s, b), __builtin_fmaf(o01[1], s, b));
  out[2] = pack_bf16x2(__builtin_fmaf(e23[0], s, b), __builtin_fmaf(o23[0], s, b));
  out[3] = pack_bf16x2(__builtin_fmaf(e23[1], s, b), __builtin_fmaf(o23[1], s, b));
}

// INT4 dequantization of one packed word (8 two's-complement nibbles) with
// bf16-valued group scale s: out[i] holds bf16(q_2i * s), bf16(q_2i+1 * s).
//
// Two v_bitop3_b32 split the word into bytes holding u = n ^ 8 = q + 8 (the
// offset-binary nibble): ((w & 0x0F0F0F0F) ^ 0x08080808) for the even
// nibbles, the same on w >> 4 for the odd ones.  dq_u4_bytes turns the bytes
// into exact floats two at a time, fma(u, s, -8 s) = (u - 8) * s = q * s is
// exact (-8 s is exact and q * s has at most 11 significant bits), and one RNE
// conversion per pair makes bf16(q * s).  Exact in value for 0 < s <= 2^120;
// for s <= 0 a zero product may come out as +0 instead of -0.
__device__ __forceinline__ void dq_int4_word(uint32_t w, float s, uint32_t out[4]) {
  // truth table of (S0 & S1) ^ S2 with S0 = 0xF0, S1 = 0xCC, S2 = 0xAA
  constexpr uint8_t AND_XOR = (uint8_t)((0xF0 & 0xCC) ^ 0xAA);
  const uint32_t ue = __builtin_amdgcn_bitop3_b32(w, 0x0F0F0F0Fu, 0x08080808u, AND_XOR);
  const uint32_t uo = __builtin_amdgcn_bitop3_b32(w >> 4, 0x0F0F0F0Fu, 0x08080808u, AND_XOR);
  dq_u4_bytes(ue, uo, s, s * -8.0f, out);
}

// INT4 word -> bf16 patterns of q + 136 for its 8 codes: 136 + q = 128 + u with
// u = q + 8 the offset-binary code, and bf16(128 + u) = 0x4300 | u exactly, so
// no conversion is needed.  out[i] holds elements 2i (low half) and 2i + 1
// (high half), the element order of dq_int4_word.  v_perm places byte i of w
// (elements 2i and 2i + 1 in its low and high nibble) in byte 0 and byte i of
// w >> 4 (element 2i + 1 in its low nibble) in byte 2; one v_bitop3 keeps the
// two low nibbles, flips their top bit (u = nibble ^ 8) and sets 0x4300.
__device__ __forceinline__ void dq_int4_word_o136(uint32_t w, uint32_t out[4]) {
  constexpr uint8_t AND_XOR = (uint8_t)((0xF0 & 0xCC) ^ 0xAA);
  const uint32_t w4 = w >> 4;
  out[0] = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(w4, w, 0x00040000u), 0x000F000Fu, 0x43084308u, AND_XOR);
  out[1] = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(w4, w, 0x00050001u), 0x000F000Fu, 0x43084308u, AND_XOR);
  out[2] = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(w4, w, 0x00060002u), 0x000F000Fu, 0x43084308u, AND_XOR);
  out[3] = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(w4, w, 0x00070003u), 0x000F000Fu, 0x43084308u, AND_XOR);
}
// bf16 patterns of -136 (two per word), the offset's correction operand.
constexpr uint32_t kBf16Neg136x2 = 0xC308C308u;

// A bf16 INT4 scale whose significand has at most 5 significant bits (3
// trailing zero mantissa bits) and whose magnitude is below 2^124: every
// product q * s with q in [-8, 7] is then a finite bf16 value, computed
// exactly, so bf16(q * s) = q * s.
__device__ __forceinline__ bool int4_scale_short(uint32_t bits16) {
  return (bits16 & 7u) == 0u && (bits16 & 0x7F80u) <= 0x7D00u;
}

// Unsigned INT4 word (8 codes q in [0, 15]) with scale s and bias b = -z * s:
// fma(q, s, b) = (q - z) * s exactly (both products have at most 12
// significant bits for a bf16 s and z <= 15), then one RNE conversion per
// pair.  Exact for 0 < s <= 2^120.
__device__ __forceinline__ void dq_uint4_word(uint32_t w, float s, float b, uint32_t out[4]) {
  dq_u4_bytes(w & 0x0F0F0F0Fu, (w >> 4) & 0x0F0F0F0Fu, s, b, out);
}

// Same result for any finite s: the magic-constant route above needs
// 15 * s to stay finite, and for s <= 0 it would give +0 where q * s is -0,
// so those scales take the direct route (sign-extend each nibble, exact fp32
// product q * s, one RNE conversion).
__device__ __forceinline__ void dq_int4_word_direct(uint32_t w, float s, uint32_t out[4]) {
  float e[8];
#pragma unroll
  for (int j = 0; j < 8; j++) e[j] = (float)(((int32_t)(w << (28 - 4 * j))) >> 28) * s;
#pragma unroll
  for (int j = 0; j < 4; j++) out[j] = pack_bf16x2(e[2 * j], e[2 * j + 1]);
}
__device__ __forceinline__ bool int4_scale_fast(float s) { return s > 0.0f && s <= 0x1p120f; }

// E2M1 word (8 codes) with E8M0 scale operand -> 4 bf16 pairs.
__device__ __forceinline__ void dq_fp4_word(uint32_t w, float sc, uint32_t out[4]) {
  out[0] = dq_fp4_pair<0>(w, sc);
  out[1] = dq_fp4_pair<1>(w, sc);
  out[2] = dq_fp4_pair<2>(w, sc);
  out[3] = dq_fp4_pair<3>(w, sc);
}

// Correctly rounded fp32 quotient x / s given y = RN(1/s), for s in
// [2^-90, 2^90] (Markstein's correction step: with y within half an ulp of 1/s
// and q within one ulp of x/s, RN(q + (x - q s) y) = RN(x / s); the remainder is
// exact through the fma).  Quotients whose magnitude is below 2^-11 may be off
// by an ulp, which cannot change an E4M3 code (they all round to 0).  The
// quotient takes the sign of x (s > 0): the correction step would otherwise
// turn x = -0 into +0 (it adds +0 and -0).
__device__ __forceinline__ float div_rn_markstein(float x, float s, float y) {
  const float q = x * y;
  const float r = __builtin_fmaf(-q, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
}

__device__ __forceinline__ float clamp448(float v) { return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f); }

// Two fp32 -> E4M3 byte pair written into half HI of `old` (no saturation: the
// inputs must already lie in [-464, 464]).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Two fp32 -> E2M1 pair of v / 2^(c-127) into byte SEL of `old`.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float a, float b, float scale_as_e8m0) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale_as_e8m0, SEL);
}

// Loads of 8 consecutive input elements as fp32 (bf16 inputs widened exactly).
__device__ __forceinline__ void load8_f32(const float* p, float v[8]) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p + 4);
  v[0] = __uint_as_float(a[0]); v[1] = __uint_as_float(a[1]); v[2] = __uint_as_float(a[2]); v[3] = __uint_as_float(a[3]);
  v[4] = __uint_as_float(b[0]); v[5] = __uint_as_float(b[1]); v[6] = __uint_as_float(b[2]); v[7] = __uint_as_float(b[3]);
}
__device__ __forceinline__ void load8_bf16(const uint16_t* p, float v[8]) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = bf16_lo(a[i]);
    v[2 * i + 1] = bf16_hi(a[i]);
  }
}
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float v[8]) {
  if constexpr (BF16) load8_bf16(reinterpret_cast<const uint16_t*>(base) + idx, v);
  else load8_f32(reinterpret_cast<const float*>(base) + idx, v);
}

__device__ __forceinline__ float absmax8(const float v[8]) {
  float m = __builtin_fabsf(v[0]);
#pragma unroll
  for (int i = 1; i < 8; i++) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  return m;
}

// Max over aligned groups of `width` consecutive lanes (width a power of two <= 64).
__device__ __forceinline__ float group_max(float v, int width) {
  for (int off = 1; off < width; off <<= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// 16-byte load through a generic pointer (LDS or global).
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// ---------------------------------------------------------------------------
// Buffer resources and direct-to-LDS loads
// ---------------------------------------------------------------------------
// Raw buffer resources: loads past `bytes` return zeros, which pads the rows
// beyond N and the x rows beyond M without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t lim = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0LL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)lim, 0x00020000);
}
__device__ __forceinline__ u32x4_t bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// soff: a wave-uniform byte offset added to voff (an SGPR operand, which
// keeps per-step constants out of the vector ALU)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t voff,
                                          uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, (int)voff,
                                           (int)soff, 0, 0);
}
// s_waitcnt with vmcnt <= n, other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the pipelined GEMM loops, without the memory fence of
// __syncthreads(): that fence would also wait for the tile loads just issued
// for later steps.  The waits the pipeline needs are explicit (vmcnt for this
// wave's tile loads before the call, and here lgkmcnt for its LDS reads), and
// the memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void tile_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace wq

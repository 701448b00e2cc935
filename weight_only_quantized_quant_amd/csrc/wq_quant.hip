// Block-scaled quantizers (fp32/bf16 -> E4M3, MXFP4, MX with a choice of scale
// rule and E2M1 or E4M3 elements, NVFP4, symmetric and asymmetric INT4) and
// the dequantizer
// entry point, for gfx950.  Memory-bound: every thread moves 16-byte vectors;
// block maxima are reduced across the lanes that share a block with xor
// shuffles.
#include <hip/hip_runtime.h>

#include "wq.h"
#include "wq_device.h"
#include "wq_host.h"

using namespace wq;

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// E4M3
// ---------------------------------------------------------------------------

// Plain cast: 8 elements per thread.  NaN -> 0x7F | sign, |x| >= 448 -> +-448.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_e4m3_cast(const void* __restrict__ x, int64_t nchunks,
                                                       uint8_t* __restrict__ codes) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= nchunks) return;
  float v[8];
  load8<BF16>(x, t * 8, v);
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    float c[4];
#pragma unroll
    for (int i = 0; i < 4; i++) c[i] = clamp448(v[4 * h + i]);
    uint32_t r = e4m3_pack2<false>(c[0], c[1], 0u);
    r = e4m3_pack2<true>(c[2], c[3], r);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float a = v[4 * h + i];
      if (a != a) {
        const uint32_t nanc = 0x7Fu | ((__float_as_uint(a) >> 24) & 0x80u);
        r = (r & ~(0xFFu << (8 * i))) | (nanc << (8 * i));
      }
    }
    w[h] = r;
  }
  *reinterpret_cast<u32x2_t*>(codes + t * 8) = u32x2_t{w[0], w[1]};
}

// One fp32 scale per 1 x block group; 16 elements per thread, block/16 lanes
// per group (groups are aligned on lanes because block divides 64*16).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_e4m3_block(const void* __restrict__ x, int64_t nchunks,
                                                        int lanes_per_block, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool valid = t0 < nchunks;            // a whole group is valid or not
  const int64_t t = valid ? t0 : nchunks - 1;
  float v[16];
  load8<BF16>(x, t * 16, v);
  load8<BF16>(x, t * 16 + 8, v + 8);
  float m = __builtin_fmaxf(absmax8(v), absmax8(v + 8));
  m = group_max(m, lanes_per_block);
  float s = m / 448.0f;                       // IEEE division
  if (s == 0.0f) s = 1.0f;
  const float y = 1.0f / s;
  const bool fast = s >= 0x1p-90f && s <= 0x1p90f;
  float q[16];
  if (fast) {
#pragma unroll
    for (int i = 0; i < 16; i++) q[i] = div_rn_markstein(v[i], s, y);
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) q[i] = clamp448(v[i] / s);
  }
  u32x4_t out;
#pragma unroll
  for (int d = 0; d < 4; d++) {
    uint32_t r = e4m3_pack2<false>(q[4 * d], q[4 * d + 1], 0u);
    out[d] = e4m3_pack2<true>(q[4 * d + 2], q[4 * d + 3], r);
  }
  if (valid) {
    *reinterpret_cast<u32x4_t*>(codes + t * 16) = out;
    if ((threadIdx.x & (lanes_per_block - 1)) == 0) scales[t / lanes_per_block] = s;
  }
}

// One fp32 scale per row: one workgroup per row, two passes over the row.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_e4m3_row(const void* __restrict__ x, int64_t cols,
                                                      uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[kThreads / 64];
  const int64_t row = blockIdx.x;
  const int64_t base = row * cols;
  float m = 0.0f;
  for (int64_t c = threadIdx.x * 8; c < cols; c += kThreads * 8) {
    float v[8];
    load8<BF16>(x, base + c, v);
    m = __builtin_fmaxf(m, absmax8(v));
  }
  m = group_max(m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  float s = m / 448.0f;
  if (s == 0.0f) s = 1.0f;
  const float y = 1.0f / s;
  const bool fast = s >= 0x1p-90f && s <= 0x1p90f;
  for (int64_t c = threadIdx.x * 8; c < cols; c += kThreads * 8) {
    float v[8];
    load8<BF16>(x, base + c, v);
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; i++) q[i] = fast ? div_rn_markstein(v[i], s, y) : clamp448(v[i] / s);
    uint32_t r0 = e4m3_pack2<true>(q[2], q[3], e4m3_pack2<false>(q[0], q[1], 0u));
    uint32_t r1 = e4m3_pack2<true>(q[6], q[7], e4m3_pack2<false>(q[4], q[5], 0u));
    *reinterpret_cast<u32x2_t*>(codes + base + c) = u32x2_t{r0, r1};
  }
  if (threadIdx.x == 0) scales[row] = s;
}

// The same for rows of at most R * 2048 elements: every thread loads its R
// pieces of 8 at once and keeps them in registers for the quantization, so
// the row is read once and the loads are all in flight together.
template <bool BF16, int R>
__global__ __launch_bounds__(kThreads) void k_e4m3_row_reg(const void* __restrict__ x, int64_t cols,
                                                          uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[kThreads / 64];
  const int64_t row = blockIdx.x;
  const int64_t base = row * cols;
  float v[R][8];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int64_t c = (int64_t)(r * kThreads + threadIdx.x) * 8;
    if (c < cols) {
      load8<BF16>(x, base + c, v[r]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) v[r][i] = 0.0f;
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < R; r++) m = __builtin_fmaxf(m, absmax8(v[r]));
  m = group_max(m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  float s = m / 448.0f;
  if (s == 0.0f) s = 1.0f;
  const float y = 1.0f / s;
  const bool fast = s >= 0x1p-90f && s <= 0x1p90f;
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int64_t c = (int64_t)(r * kThreads + threadIdx.x) * 8;
    if (c < cols) {
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; i++) q[i] = fast ? div_rn_markstein(v[r][i], s, y) : clamp448(v[r][i] / s);
      uint32_t r0 = e4m3_pack2<true>(q[2], q[3], e4m3_pack2<false>(q[0], q[1], 0u));
      uint32_t r1 = e4m3_pack2<true>(q[6], q[7], e4m3_pack2<false>(q[4], q[5], 0u));
      *reinterpret_cast<u32x2_t*>(codes + base + c) = u32x2_t{r0, r1};
    }
  }
  if (threadIdx.x == 0) scales[row] = s;
}

// ---------------------------------------------------------------------------
// MXFP4: 16 elements per thread; block 32 -> lane pairs, block 16 -> one lane.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_mxfp4(const void* __restrict__ x, int64_t nchunks, int block,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool valid = t0 < nchunks;
  const int64_t t = valid ? t0 : nchunks - 1;
  float v[16];
  load8<BF16>(x, t * 16, v);
  load8<BF16>(x, t * 16 + 8, v + 8);
  float m = __builtin_fmaxf(absmax8(v), absmax8(v + 8));
  if (block == 32) m = __builtin_fmaxf(m, __shfl_xor(m, 1, 64));
  const uint32_t code = e8m0_code(m);
  const float sc = e8m0_as_scale(code);
  uint32_t w0 = e2m1_pack2<0>(0u, v[0], v[1], sc);
  w0 = e2m1_pack2<1>(w0, v[2], v[3], sc);
  w0 = e2m1_pack2<2>(w0, v[4], v[5], sc);
  w0 = e2m1_pack2<3>(w0, v[6], v[7], sc);
  uint32_t w1 = e2m1_pack2<0>(0u, v[8], v[9], sc);
  w1 = e2m1_pack2<1>(w1, v[10], v[11], sc);
  w1 = e2m1_pack2<2>(w1, v[12], v[13], sc);
  w1 = e2m1_pack2<3>(w1, v[14], v[15], sc);
  if (valid) {
    *reinterpret_cast<u32x2_t*>(codes + t * 8) = u32x2_t{w0, w1};
    if (block == 16) scales[t] = (uint8_t)code;
    else if ((threadIdx.x & 1) == 0) scales[t >> 1] = (uint8_t)code;
  }
}

// ---------------------------------------------------------------------------
// MX block quantizer with a selectable E8M0 rule and E2M1 or E4M3 elements.
// Same thread layout as k_mxfp4: 16 elements per thread, lane pairs for block 32.
// ---------------------------------------------------------------------------

// E8M0 code of a block maximum.  Exponent rules add an increment to the fp32
// pattern (the sum stays below 2^31 for finite input), take the biased
// exponent and subtract the element format's top binade (2 for E2M1, 8 for
// E4M3).  The division rules take the exponent of an fp32 quotient by the
// element maximum: floor via a multiply by its fp32 reciprocal, ceil via a
// correctly rounded division, rounded up to a power of two exactly (a nonzero
// fraction adds one; a subnormal quotient above 2^-127 gives 1).
template <bool E4M3>
__device__ __forceinline__ uint32_t mx_code(float vmax, int rule) {
  constexpr uint32_t kOff = E4M3 ? 8u : 2u;
  const uint32_t bits = __float_as_uint(vmax) & 0x7FFFFFFFu;
  const float a = __uint_as_float(bits);
  if (rule == WQ_MX_FLOOR_DIV) return __float_as_uint(a * (E4M3 ? 1.0f / 448.0f : 1.0f / 6.0f)) >> 23;
  if (rule == WQ_MX_CEIL_DIV) {
    const uint32_t qb = __float_as_uint(a / (E4M3 ? 448.0f : 6.0f));
    const uint32_t be = qb >> 23;
    return be ? be + ((qb & 0x7FFFFFu) != 0u) : (uint32_t)(qb > 0x400000u);
  }
  const uint32_t inc = rule == WQ_MX_ROUND ? (E4M3 ? 1u << 19 : 1u << 21) : (rule == WQ_MX_HALF ? 1u << 22 : 0u);
  const uint32_t be = (bits + inc) >> 23;
  return be > kOff ? be - kOff : 0u;
}

template <bool BF16, bool E4M3>
__global__ __launch_bounds__(kThreads) void k_mx(const void* __restrict__ x, int64_t nchunks, int block, int rule,
                                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool valid = t0 < nchunks;
  const int64_t t = valid ? t0 : nchunks - 1;
  float v[16];
  load8<BF16>(x, t * 16, v);
  load8<BF16>(x, t * 16 + 8, v + 8);
  float m = __builtin_fmaxf(absmax8(v), absmax8(v + 8));
  if (block == 32) m = __builtin_fmaxf(m, __shfl_xor(m, 1, 64));
  const uint32_t code = mx_code<E4M3>(m, rule);
  if constexpr (E4M3) {
    // x * 2^(127 - c) is exact (or underflows far below the E4M3 grid); the
    // clamp saturates what lies above 448 before the RNE conversion
    const int sh = 127 - (int)code;
    float q[16];
#pragma unroll
    for (int i = 0; i < 16; i++) q[i] = clamp448(__builtin_ldexpf(v[i], sh));
    u32x4_t out;
#pragma unroll
    for (int d = 0; d < 4; d++) {
      uint32_t r = e4m3_pack2<false>(q[4 * d], q[4 * d + 1], 0u);
      out[d] = e4m3_pack2<true>(q[4 * d + 2], q[4 * d + 3], r);
    }
    if (valid) *reinterpret_cast<u32x4_t*>(codes + t * 16) = out;
  } else {
    const float sc = e8m0_as_scale(code);
    uint32_t w0 = e2m1_pack2<0>(0u, v[0], v[1], sc);
    w0 = e2m1_pack2<1>(w0, v[2], v[3], sc);
    w0 = e2m1_pack2<2>(w0, v[4], v[5], sc);
    w0 = e2m1_pack2<3>(w0, v[6], v[7], sc);
    uint32_t w1 = e2m1_pack2<0>(0u, v[8], v[9], sc);
    w1 = e2m1_pack2<1>(w1, v[10], v[11], sc);
    w1 = e2m1_pack2<2>(w1, v[12], v[13], sc);
    w1 = e2m1_pack2<3>(w1, v[14], v[15], sc);
    if (valid) *reinterpret_cast<u32x2_t*>(codes + t * 8) = u32x2_t{w0, w1};
  }
  if (valid) {
    if (block == 16) scales[t] = (uint8_t)code;
    else if ((threadIdx.x & 1) == 0) scales[t >> 1] = (uint8_t)code;
  }
}

// ---------------------------------------------------------------------------
// NVFP4: one 16-element block per thread.  Block scale e4m3(RN(RN(amax/6)/g))
// (two correctly rounded divisions), elements RN(x / d) with d = e4m3 value * g
// the dequantized scale, clamped to +-6 and converted with an unscaled E2M1
// conversion (quotients beyond 16 only need their sign).  A zero d gives zeros
// with the sign of x.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_nvfp4(const void* __restrict__ x, int64_t nblocks, float g,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= nblocks) return;
  float v[16];
  load8<BF16>(x, t * 16, v);
  load8<BF16>(x, t * 16 + 8, v + 8);
  const float m = __builtin_fmaxf(absmax8(v), absmax8(v + 8));
  const float sq = (m / 6.0f) / g;
  const uint32_t s8 = e4m3_pack2<false>(clamp448(sq), 0.0f, 0u) & 0xFFu;
  const float d = bf16_lo(dq_fp8_pair<false>(s8)) * g;
  float q[16];
  if (d >= 0x1p-90f && d <= 0x1p90f) {
    // a saturated scale can leave quotients far above 6 (even past fp32): the
    // first estimate decides those (the correction step would turn an
    // infinite estimate into NaN)
    const float y = 1.0f / d;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const float q0 = v[i] * y;
      q[i] = __builtin_fabsf(q0) > 16.0f ? q0 : div_rn_markstein(v[i], d, y);
    }
  } else if (d > 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; i++) q[i] = v[i] / d;
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) q[i] = __builtin_copysignf(0.0f, v[i]);
  }
#pragma unroll
  for (int i = 0; i < 16; i++) q[i] = __builtin_fminf(__builtin_fmaxf(q[i], -6.0f), 6.0f);
  uint32_t w0 = e2m1_pack2<0>(0u, q[0], q[1], 1.0f);
  w0 = e2m1_pack2<1>(w0, q[2], q[3], 1.0f);
  w0 = e2m1_pack2<2>(w0, q[4], q[5], 1.0f);
  w0 = e2m1_pack2<3>(w0, q[6], q[7], 1.0f);
  uint32_t w1 = e2m1_pack2<0>(0u, q[8], q[9], 1.0f);
  w1 = e2m1_pack2<1>(w1, q[10], q[11], 1.0f);
  w1 = e2m1_pack2<2>(w1, q[12], q[13], 1.0f);
  w1 = e2m1_pack2<3>(w1, q[14], q[15], 1.0f);
  *reinterpret_cast<u32x2_t*>(codes + t * 8) = u32x2_t{w0, w1};
  scales[t] = (uint8_t)s8;
}

// ---------------------------------------------------------------------------
// INT4 symmetric groups: 16 elements per thread, group/16 lanes per group.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_int4(const void* __restrict__ x, int64_t nchunks,
                                                  int lanes_per_group, uint32_t* __restrict__ packed,
                                                  uint16_t* __restrict__ scales) {
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool valid = t0 < nchunks;
  const int64_t t = valid ? t0 : nchunks - 1;
  float v[16];
  load8<BF16>(x, t * 16, v);
  load8<BF16>(x, t * 16 + 8, v + 8);
  float m = __builtin_fmaxf(absmax8(v), absmax8(v + 8));
  m = group_max(m, lanes_per_group);
  // RN_f32(amax / 7) rounded to a 5-bit significand, ties to even: the fp32
  // pattern rounded at mantissa bit 19 (a carry moves into the exponent), which
  // is a bf16 value with 3 trailing zero mantissa bits, so that q * s is exact
  // in bf16 for every code
  const uint32_t qb = __float_as_uint(m / 7.0f);
  uint32_t sb = ((qb + 0x3FFFFu + ((qb >> 19) & 1u)) & 0xFFF80000u) >> 16;
  if ((sb & 0x7FFFu) == 0u) sb = 0x3F80u;
  const float s = bf16_to_f32(sb);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; i++) {
    float q = __builtin_rintf(v[i] / s);      // IEEE division, then ties-to-even
    q = __builtin_fminf(__builtin_fmaxf(q, -8.0f), 7.0f);
    const uint32_t nib = (uint32_t)((int)q) & 0xFu;
    w[i >> 3] |= nib << (4 * (i & 7));
  }
  if (valid) {
    *reinterpret_cast<u32x2_t*>(packed + t * 2) = u32x2_t{w[0], w[1]};
    if ((threadIdx.x & (lanes_per_group - 1)) == 0) scales[t / lanes_per_group] = (uint16_t)sb;
  }
}

// ---------------------------------------------------------------------------
// Dequantization to bf16: 8 elements (one 16-byte output) per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_dq_int4(const uint32_t* __restrict__ packed,
                                                     const uint16_t* __restrict__ scales, int64_t nchunks,
                                                     int64_t K, int group, uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= nchunks) return;
  const int64_t e = t * 8, n = e / K, k = e % K;
  const float s = bf16_to_f32(scales[n * (K / group) + k / group]);
  uint32_t o[4];
  if (int4_scale_fast(s)) dq_int4_word(packed[t], s, o);
  else dq_int4_word_direct(packed[t], s, o);
  *reinterpret_cast<u32x4_t*>(out + e) = u32x4_t{o[0], o[1], o[2], o[3]};
}

__global__ __launch_bounds__(kThreads) void k_dq_fp4(const uint32_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales, int64_t nchunks, int64_t K,
                                                    int block, uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= nchunks) return;
  const int64_t e = t * 8, n = e / K, k = e % K;
  const float sc = e8m0_as_scale(scales[n * (K / block) + k / block]);
  uint32_t o[4];
  dq_fp4_word(codes[t], sc, o);
  *reinterpret_cast<u32x4_t*>(out + e) = u32x4_t{o[0], o[1], o[2], o[3]};
}

// NVFP4 operand: E2M1 word times its block's E4M3 scale value (exact in bf16).
__global__ __launch_bounds__(kThreads) void k_dq_nv4(const uint32_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales, int64_t nchunks, int64_t K,
                                                    uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= nchunks) return;
  const int64_t e = t * 8, n = e / K, k = e % K;
  const float sc = bf16_lo(dq_fp8_pair<false>(scales[n * (K / 16) + k / 16]));
  uint32_t o[4];
  dq_nv4_word(codes[t], sc, o);
  *reinterpret_cast<u32x4_t*>(out + e) = u32x4_t{o[0], o[1], o[2], o[3]};
}

__global__ __launch_bounds__(kThreads) void k_dq_fp8(const u32x2_t* __restrict__ codes, int64_t nchunks,
                                                    uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= nchunks) return;
  const u32x2_t w = codes[t];
  u32x4_t o{dq_fp8_pair<false>(w[0]), dq_fp8_pair<true>(w[0]), dq_fp8_pair<false>(w[1]), dq_fp8_pair<true>(w[1])};
  *reinterpret_cast<u32x4_t*>(out + t * 8) = o;
}

// ---------------------------------------------------------------------------
// Asymmetric INT4: 16 elements per thread, group/16 lanes per group.  Range
// [min(min x, 0), max(max x, 0)], s = bf16(RN(RN(hi - lo) / 15)) (1 if zero),
// z = clamp(rint(RN(-lo / s)), 0, 15), q = clamp(rint(RN(x / s)) + z, 0, 15);
// one word per group holds the scale bits (low half) and z (bits 16..23).
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_int4_asym(const void* __restrict__ x, int64_t nchunks,
                                                       int lanes_per_group, uint32_t* __restrict__ packed,
                                                       uint32_t* __restrict__ scalezero) {
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool valid = t0 < nchunks;
  const int64_t t = valid ? t0 : nchunks - 1;
  float v[16];
  load8<BF16>(x, t * 16, v);
  load8<BF16>(x, t * 16 + 8, v + 8);
  float hi = 0.0f, nlo = 0.0f;                 // max(x, 0) and max(-x, 0)
#pragma unroll
  for (int i = 0; i < 16; i++) {
    hi = __builtin_fmaxf(hi, v[i]);
    nlo = __builtin_fmaxf(nlo, -v[i]);
  }
  hi = group_max(hi, lanes_per_group);
  nlo = group_max(nlo, lanes_per_group);
  uint32_t sb = f32_to_bf16_bits((hi + nlo) / 15.0f);   // hi - lo with lo = -nlo
  if ((sb & 0x7FFFu) == 0u) sb = 0x3F80u;
  const float s = bf16_to_f32(sb);
  const float z = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(nlo / s), 0.0f), 15.0f);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; i++) {
    float q = __builtin_rintf(v[i] / s) + z;
    q = __builtin_fminf(__builtin_fmaxf(q, 0.0f), 15.0f);
    w[i >> 3] |= ((uint32_t)q) << (4 * (i & 7));
  }
  if (valid) {
    *reinterpret_cast<u32x2_t*>(packed + t * 2) = u32x2_t{w[0], w[1]};
    if ((threadIdx.x & (lanes_per_group - 1)) == 0) scalezero[t / lanes_per_group] = sb | ((uint32_t)z << 16);
  }
}

// (q - z) * s of a word of unsigned codes, from one scale-zero word per group.
__global__ __launch_bounds__(kThreads) void k_dq_uint4(const uint32_t* __restrict__ packed,
                                                      const uint32_t* __restrict__ scalezero, int64_t nchunks,
                                                      int64_t K, int group, uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= nchunks) return;
  const int64_t e = t * 8, n = e / K, k = e % K;
  const uint32_t sz = scalezero[n * (K / group) + k / group];
  const float s = bf16_to_f32(sz & 0xFFFFu);
  uint32_t o[4];
  dq_uint4_word(packed[t], s, -(float)((sz >> 16) & 0xFFu) * s, o);
  *reinterpret_cast<u32x4_t*>(out + e) = u32x4_t{o[0], o[1], o[2], o[3]};
}

inline unsigned grid_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

extern "C" {

wq_status quantize_e4m3(const void* x, int x_dtype, int64_t rows, int64_t cols, int32_t block, uint8_t* codes,
                        float* scales, void* stream) {
  if (!x || !codes || rows <= 0 || cols <= 0 || cols % 8) return WQ_EINVAL;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16) return WQ_EUNSUPPORTED;
  if (!wq_numel_ok(rows, cols)) return WQ_EINVAL;
  if (!wq_aligned(x) || !wq_aligned(codes) || (scales && !wq_aligned(scales))) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = x_dtype == WQ_BF16;
  const int64_t n = rows * cols;
  if (block == 0) {
    const int64_t nch = n / 8;
    if (bf) k_e4m3_cast<true><<<grid_for(nch), kThreads, 0, s>>>(x, nch, codes);
    else k_e4m3_cast<false><<<grid_for(nch), kThreads, 0, s>>>(x, nch, codes);
    return wq_launch_status();
  }
  if (!scales) return WQ_EINVAL;
  if (block == -1) {
    if (rows > 0x7FFFFFFF) return WQ_EINVAL;
    const unsigned g = (unsigned)rows;
    constexpr int64_t PIECE = kThreads * 8;            // elements per register round of a row
    if (cols <= PIECE) {
      if (bf) k_e4m3_row_reg<true, 1><<<g, kThreads, 0, s>>>(x, cols, codes, scales);
      else k_e4m3_row_reg<false, 1><<<g, kThreads, 0, s>>>(x, cols, codes, scales);
    } else if (cols <= 2 * PIECE) {
      if (bf) k_e4m3_row_reg<true, 2><<<g, kThreads, 0, s>>>(x, cols, codes, scales);
      else k_e4m3_row_reg<false, 2><<<g, kThreads, 0, s>>>(x, cols, codes, scales);
    } else if (cols <= 4 * PIECE) {
      if (bf) k_e4m3_row_reg<true, 4><<<g, kThreads, 0, s>>>(x, cols, codes, scales);
      else k_e4m3_row_reg<false, 4><<<g, kThreads, 0, s>>>(x, cols, codes, scales);
    } else {
      if (bf) k_e4m3_row<true><<<g, kThreads, 0, s>>>(x, cols, codes, scales);
      else k_e4m3_row<false><<<g, kThreads, 0, s>>>(x, cols, codes, scales);
    }
    return wq_launch_status();
  }
  if (block != 16 && block != 32 && block != 64 && block != 128 && block != 256) return WQ_EUNSUPPORTED;
  if (cols % block) return WQ_EINVAL;
  const int64_t nch = n / 16;
  const int lpb = block / 16;
  if (bf) k_e4m3_block<true><<<grid_for(nch), kThreads, 0, s>>>(x, nch, lpb, codes, scales);
  else k_e4m3_block<false><<<grid_for(nch), kThreads, 0, s>>>(x, nch, lpb, codes, scales);
  return wq_launch_status();
}

wq_status quantize_mxfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, int32_t block, uint8_t* codes,
                         uint8_t* scales, void* stream) {
  if (!x || !codes || !scales || rows <= 0 || cols <= 0) return WQ_EINVAL;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16) return WQ_EUNSUPPORTED;
  if (block != 16 && block != 32) return WQ_EUNSUPPORTED;
  if (cols % 32 || !wq_numel_ok(rows, cols)) return WQ_EINVAL;
  if (!wq_aligned(x) || !wq_aligned(codes) || !wq_aligned(scales)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nch = rows * cols / 16;
  if (x_dtype == WQ_BF16) k_mxfp4<true><<<grid_for(nch), kThreads, 0, s>>>(x, nch, block, codes, scales);
  else k_mxfp4<false><<<grid_for(nch), kThreads, 0, s>>>(x, nch, block, codes, scales);
  return wq_launch_status();
}

wq_status quantize_mx(const void* x, int x_dtype, int64_t rows, int64_t cols, int32_t block, int32_t elem,
                      int32_t rule, uint8_t* codes, uint8_t* scales, void* stream) {
  if (!x || !codes || !scales || rows <= 0 || cols <= 0) return WQ_EINVAL;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16) return WQ_EUNSUPPORTED;
  if (elem != WQ_E2M1X2 && elem != WQ_E4M3) return WQ_EUNSUPPORTED;
  if (rule < WQ_MX_ROUND || rule > WQ_MX_CEIL_DIV) return WQ_EINVAL;
  if (block != 16 && block != 32) return WQ_EUNSUPPORTED;
  if (cols % 32 || !wq_numel_ok(rows, cols)) return WQ_EINVAL;
  if (!wq_aligned(x) || !wq_aligned(codes) || !wq_aligned(scales)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nch = rows * cols / 16;
  const unsigned g = grid_for(nch);
  const bool bf = x_dtype == WQ_BF16;
  if (elem == WQ_E4M3) {
    if (bf) k_mx<true, true><<<g, kThreads, 0, s>>>(x, nch, block, rule, codes, scales);
    else k_mx<false, true><<<g, kThreads, 0, s>>>(x, nch, block, rule, codes, scales);
  } else {
    if (bf) k_mx<true, false><<<g, kThreads, 0, s>>>(x, nch, block, rule, codes, scales);
    else k_mx<false, false><<<g, kThreads, 0, s>>>(x, nch, block, rule, codes, scales);
  }
  return wq_launch_status();
}

wq_status quantize_nvfp4(const void* x, int x_dtype, int64_t rows, int64_t cols, float tensor_scale,
                         uint8_t* codes, uint8_t* scales, void* stream) {
  if (!x || !codes || !scales || rows <= 0 || cols <= 0 || cols % 16) return WQ_EINVAL;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16) return WQ_EUNSUPPORTED;
  if (!(tensor_scale > 0.0f) || !(tensor_scale <= 3.4028234e38f)) return WQ_EINVAL;
  if (!wq_numel_ok(rows, cols)) return WQ_EINVAL;
  if (!wq_aligned(x) || !wq_aligned(codes) || !wq_aligned(scales)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nb = rows * cols / 16;
  if (x_dtype == WQ_BF16) k_nvfp4<true><<<grid_for(nb), kThreads, 0, s>>>(x, nb, tensor_scale, codes, scales);
  else k_nvfp4<false><<<grid_for(nb), kThreads, 0, s>>>(x, nb, tensor_scale, codes, scales);
  return wq_launch_status();
}

wq_status quantize_int4(const void* w, int w_dtype, int64_t rows, int64_t cols, int32_t group, uint32_t* packed,
                        uint16_t* scales, void* stream) {
  if (!w || !packed || !scales || rows <= 0 || cols <= 0) return WQ_EINVAL;
  if (w_dtype != WQ_F32 && w_dtype != WQ_BF16) return WQ_EUNSUPPORTED;
  if (group != 32 && group != 64 && group != 128) return WQ_EUNSUPPORTED;
  if (cols % group || cols % 32 || !wq_numel_ok(rows, cols)) return WQ_EINVAL;
  if (!wq_aligned(w) || !wq_aligned(packed) || !wq_aligned(scales)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nch = rows * cols / 16;
  const int lpg = group / 16;
  if (w_dtype == WQ_BF16) k_int4<true><<<grid_for(nch), kThreads, 0, s>>>(w, nch, lpg, packed, scales);
  else k_int4<false><<<grid_for(nch), kThreads, 0, s>>>(w, nch, lpg, packed, scales);
  return wq_launch_status();
}

wq_status quantize_int4_asym(const void* w, int w_dtype, int64_t rows, int64_t cols, int32_t group,
                             uint32_t* packed, uint32_t* scalezero, void* stream) {
  if (!w || !packed || !scalezero || rows <= 0 || cols <= 0) return WQ_EINVAL;
  if (w_dtype != WQ_F32 && w_dtype != WQ_BF16) return WQ_EUNSUPPORTED;
  if (group != 32 && group != 64 && group != 128) return WQ_EUNSUPPORTED;
  if (cols % group || !wq_numel_ok(rows, cols)) return WQ_EINVAL;
  if (!wq_aligned(w) || !wq_aligned(packed) || !wq_aligned(scalezero)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nch = rows * cols / 16;
  const int lpg = group / 16;
  if (w_dtype == WQ_BF16) k_int4_asym<true><<<grid_for(nch), kThreads, 0, s>>>(w, nch, lpg, packed, scalezero);
  else k_int4_asym<false><<<grid_for(nch), kThreads, 0, s>>>(w, nch, lpg, packed, scalezero);
  return wq_launch_status();
}

wq_status wq_dequant(const void* wqp, int w_dtype, const void* w_scales, int s_dtype, int32_t group, int64_t N,
                     int64_t K, uint16_t* w_bf16, void* stream) {
  if (!wqp || !w_bf16 || N <= 0 || K <= 0 || K % 32 || !wq_numel_ok(N, K)) return WQ_EINVAL;
  if (!wq_aligned(wqp) || !wq_aligned(w_bf16)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nch = N * K / 8;
  if (w_dtype == WQ_INT4X8) {
    if (s_dtype != WQ_BF16 || (group != 32 && group != 64 && group != 128)) return WQ_EUNSUPPORTED;
    if (!w_scales) return WQ_EINVAL;
    if (K % group) return WQ_EINVAL;
    k_dq_int4<<<grid_for(nch), kThreads, 0, s>>>((const uint32_t*)wqp, (const uint16_t*)w_scales, nch, K, group,
                                                  w_bf16);
    return wq_launch_status();
  }
  if (w_dtype == WQ_UINT4X8) {
    if (s_dtype != WQ_BF16Z || (group != 32 && group != 64 && group != 128)) return WQ_EUNSUPPORTED;
    if (!w_scales) return WQ_EINVAL;
    if (K % group) return WQ_EINVAL;
    k_dq_uint4<<<grid_for(nch), kThreads, 0, s>>>((const uint32_t*)wqp, (const uint32_t*)w_scales, nch, K, group,
                                                   w_bf16);
    return wq_launch_status();
  }
  if (w_dtype == WQ_E2M1X2 && s_dtype == WQ_E4M3) {
    if (group != 16) return WQ_EUNSUPPORTED;
    if (!w_scales) return WQ_EINVAL;
    k_dq_nv4<<<grid_for(nch), kThreads, 0, s>>>((const uint32_t*)wqp, (const uint8_t*)w_scales, nch, K, w_bf16);
    return wq_launch_status();
  }
  if (w_dtype == WQ_E2M1X2) {
    if (s_dtype != WQ_E8M0 || (group != 16 && group != 32)) return WQ_EUNSUPPORTED;
    if (!w_scales) return WQ_EINVAL;
    k_dq_fp4<<<grid_for(nch), kThreads, 0, s>>>((const uint32_t*)wqp, (const uint8_t*)w_scales, nch, K, group,
                                                 w_bf16);
    return wq_launch_status();
  }
  if (w_dtype == WQ_E4M3) {
    if (s_dtype != WQ_F32) return WQ_EUNSUPPORTED;
    k_dq_fp8<<<grid_for(nch), kThreads, 0, s>>>((const u32x2_t*)wqp, nch, w_bf16);
    return wq_launch_status();
  }
  return WQ_EUNSUPPORTED;
}

}  // extern "C"

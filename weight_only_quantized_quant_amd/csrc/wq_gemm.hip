// Weight-only quantized matmul y[M,N] = x[M,K] . dequant(W[N,K])^T for gfx950.
//
// Decode (M <= 16): split-K GEMV.  For M <= 4 a workgroup of 4 waves owns 16
// output columns; its waves split K and stream the packed weights through a
// small LDS ring fed by direct-to-LDS loads (E4M3 weights straight into
// registers).  For 4 < M <= 16 a workgroup of 16 waves owns 64 columns and
// stages x once in LDS.  The weights are converted to bf16 in registers and
// feed v_mfma_f32_16x16x32_bf16 with the x rows as the other operand; the
// partial 16x16 tiles are reduced through LDS and rounded to bf16 once.
//
// Prefill (M > 16): 256x256 output tile per workgroup of 8 waves, K step 64,
// three LDS stages filled by direct-to-LDS loads (x in bf16, W still packed);
// each wave dequantizes its W fragments from LDS in registers right before
// v_mfma_f32_32x32x16_bf16.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wq.h"
#include "wq_device.h"
#include "wq_host.h"

using namespace wq;

namespace {

// W_NV4: E2M1 codes with an E4M3 scale per 16 elements (NVFP4).
// W_UINT4: unsigned INT4 codes with a scale-zero word per group (asymmetric).
enum { W_INT4 = 0, W_FP4 = 1, W_FP8 = 2, W_NV4 = 3, W_UINT4 = 4 };

template <int WDT> struct WTraits;
template <> struct WTraits<W_INT4> { static constexpr int bits = 4; };
template <> struct WTraits<W_FP4> { static constexpr int bits = 4; };
template <> struct WTraits<W_FP8> { static constexpr int bits = 8; };
template <> struct WTraits<W_NV4> { static constexpr int bits = 4; };
template <> struct WTraits<W_UINT4> { static constexpr int bits = 4; };

// log2 of the scale group along K (INT4: the caller's group) and bytes per scale
template <int WDT>
__host__ __device__ constexpr int gshift_of(int int4_shift) {
  return WDT == W_INT4 || WDT == W_UINT4 ? int4_shift : WDT == W_NV4 ? 4 : 5;
}
template <int WDT> constexpr int scale_bytes() { return WDT == W_INT4 ? 2 : WDT == W_UINT4 ? 4 : 1; }

// Scale operand of one lane's 32-element chunk: one value, or for NVFP4 the
// values of its two 16-element blocks.
// For asymmetric INT4: the scale and the bias -z * s.
struct Sc2 { float lo, hi; };
struct ScZ { float s, b; };
template <int WDT> struct ScaleT { using type = float; };
template <> struct ScaleT<W_NV4> { using type = Sc2; };
template <> struct ScaleT<W_UINT4> { using type = ScZ; };
template <int WDT> using scale_t = typename ScaleT<WDT>::type;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{a, b, c, d});
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Convert one packed 16-byte weight chunk to bf16 MFMA operands.
// 4-bit: 32 elements -> 4 operands of 8; 8-bit: 16 elements -> 2 operands.
template <int WDT>
__device__ __forceinline__ void dequant16(u32x4_t w, scale_t<WDT> s, bf16x8_t out[4]) {
  if constexpr (WDT == W_NV4) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t o[4];
      dq_nv4_word(w[j], j < 2 ? s.lo : s.hi, o);
      out[j] = as_bf16x8(o[0], o[1], o[2], o[3]);
    }
  } else if constexpr (WDT == W_UINT4) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t o[4];
      dq_uint4_word(w[j], s.s, s.b, o);
      out[j] = as_bf16x8(o[0], o[1], o[2], o[3]);
    }
  } else if constexpr (WDT == W_INT4) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t o[4];
      dq_int4_word(w[j], s, o);
      out[j] = as_bf16x8(o[0], o[1], o[2], o[3]);
    }
  } else if constexpr (WDT == W_FP4) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t o[4];
      dq_fp4_word(w[j], s, o);
      out[j] = as_bf16x8(o[0], o[1], o[2], o[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      out[j] = as_bf16x8(dq_fp8_pair<false>(w[2 * j]), dq_fp8_pair<true>(w[2 * j]), dq_fp8_pair<false>(w[2 * j + 1]),
                         dq_fp8_pair<true>(w[2 * j + 1]));
    }
  }
}

// One 16-byte INT4 chunk (a 128-element step inside one scale group) of a
// 16-column tile in the exact-code form, for a scale with a 5-bit significand
// (int4_scale_short): then bf16(q * s) = q * s and
//   x . bf16(q s) = s * (x . (q + 136) + x . (-136)).
// The codes go to the MFMA as the exact bf16 patterns of q + 136 (no
// conversion), a second MFMA chain against the constant -136 removes the
// offset, and the fp32 sum of the group is scaled once.  The two chains take
// the same x fragments in the same order into separate accumulators, so for
// all-zero codes they are exact negatives and the chunk adds exactly zero.
__device__ __forceinline__ void mma_int4_exact_codes(const bf16x8_t xa[4], u32x4_t wv, float s, f32x4_t& acc) {
  const bf16x8_t neg136 = as_bf16x8(kBf16Neg136x2, kBf16Neg136x2, kBf16Neg136x2, kBf16Neg136x2);
  f32x4_t pq = f32x4_t{0.f, 0.f, 0.f, 0.f}, pc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    uint32_t o[4];
    dq_int4_word_o136(wv[j], o);
    pq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], as_bf16x8(o[0], o[1], o[2], o[3]), pq, 0, 0, 0);
    pc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], neg136, pc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; i++) acc[i] = __builtin_fmaf(s, pq[i] + pc[i], acc[i]);
}

// ---------------------------------------------------------------------------
// Decode GEMV
// ---------------------------------------------------------------------------
// Scales loaded ahead of use are kept as raw bits and converted at the use:
// converting next to the load would make the wave wait for it there.
// NVFP4: idx is the first of the chunk's two blocks (even), whose two E4M3
// codes are read as one 16-bit word.
template <int WDT>
__device__ __forceinline__ uint32_t scale_raw_of(__amdgpu_buffer_rsrc_t r, uint32_t idx) {
  if constexpr (WDT == W_INT4) return __builtin_amdgcn_raw_buffer_load_b16(r, (int)(idx * 2), 0, 0);
  else if constexpr (WDT == W_FP4) return __builtin_amdgcn_raw_buffer_load_b8(r, (int)idx, 0, 0);
  else if constexpr (WDT == W_NV4) return __builtin_amdgcn_raw_buffer_load_b16(r, (int)idx, 0, 0);
  else if constexpr (WDT == W_UINT4) return __builtin_amdgcn_raw_buffer_load_b32(r, (int)(idx * 4), 0, 0);
  else return 0u;
}
template <int WDT>
__device__ __forceinline__ scale_t<WDT> scale_from_raw(uint32_t raw) {
  if constexpr (WDT == W_INT4) return bf16_to_f32(raw);
  else if constexpr (WDT == W_FP4) return e8m0_as_scale(raw);
  else if constexpr (WDT == W_NV4) {
    const uint32_t p = dq_fp8_pair<false>(raw);            // both E4M3 codes, exact in bf16
    return Sc2{bf16_lo(p), bf16_hi(p)};
  } else if constexpr (WDT == W_UINT4) {
    const float s = bf16_lo(raw);
    return ScZ{s, -(float)((raw >> 16) & 0xFFu) * s};
  } else return 1.0f;
}
template <int WDT>
__device__ __forceinline__ scale_t<WDT> scale_of(__amdgpu_buffer_rsrc_t r, uint32_t idx) {
  return scale_from_raw<WDT>(scale_raw_of<WDT>(r, idx));
}

// General decode form for M <= 4 (K not taken by the ring): one 16-column
// tile per workgroup.  Each wave stages the x rows of its own K chunk in a
// private LDS region (M x NSTEP*KSTEP bf16, one 16-byte load per lane per row)
// next to a 64-byte zero block; lanes whose MFMA row is >= M read the zero
// block.  No workgroup barrier is needed: LDS operations of one wave execute
// in order.
// Issue order per chunk: x staging loads, scales, weights.
// K splits into nchunk chunks of NSTEP steps; wave w of the S waves takes
// chunks [w nchunk / S, (w + 1) nchunk / S), so the waves' shares differ by at
// most one chunk whatever K is.
template <int WDT, int NSTEP>
__global__ __launch_bounds__(1024) void k_gemv(const uint16_t* __restrict__ x, int M, int64_t N, int64_t K,
                                             const uint8_t* __restrict__ w, const void* __restrict__ sc,
                                             int group_shift, const float* __restrict__ chscale, float alpha,
                                             uint16_t* __restrict__ y, int nchunk) {
  constexpr int EPL = WTraits<WDT>::bits == 4 ? 32 : 16;   // elements per lane per step
  constexpr int KSTEP = 4 * EPL;                            // K covered by a wave per step
  constexpr int KCH = NSTEP * KSTEP;                        // K per wave per chunk
  constexpr int MF = EPL / 8;                               // MFMAs per step per tile
  constexpr int BPE2 = WTraits<WDT>::bits == 4 ? 1 : 2;     // bytes per 2 elements
  constexpr int SB = scale_bytes<WDT>();
  constexpr int XW = 4 * KCH * 2 + 64;                      // per-wave x region (up to 4 rows)
  static_assert(KCH <= 512, "x staging uses one 16-byte chunk per lane per 512 k");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int S = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const uint32_t rowbytes = (uint32_t)(K * BPE2 / 2);
  const int64_t nrows = N - n0 < 16 ? N - n0 : 16;
  const int gs = gshift_of<WDT>(group_shift);               // log2 of the scale group
  const uint32_t spr = (uint32_t)(K >> gs);                  // scales per row
  const auto rw = make_rsrc(w + n0 * rowbytes, nrows * rowbytes);
  const auto rs = make_rsrc(reinterpret_cast<const uint8_t*>(sc) + (WDT == W_FP8 ? 0 : n0 * spr * SB),
                            WDT == W_FP8 ? 0 : nrows * spr * SB);
  const auto rx = make_rsrc(x, (int64_t)M * K * 2);
  const int c0 = (int)((int64_t)wave * nchunk / S), niter = (int)((int64_t)(wave + 1) * nchunk / S) - c0;
  const uint32_t kbase = (uint32_t)(c0 * KCH);

  uint8_t* xw = smem + wave * XW;                            // this wave's x rows, then zeros
  float* red = reinterpret_cast<float*>(smem + S * XW);
  if (lane < 4) *reinterpret_cast<u32x4_t*>(xw + 4 * KCH * 2 + 16 * lane) = u32x4_t{0u, 0u, 0u, 0u};

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < niter; it++) {
    const uint32_t k0 = kbase + (uint32_t)(it * KCH);
    // x staging: row r, 16-byte chunk `lane` of the KCH-wide slice (KCH/8 chunks <= 64)
    u32x4_t xst[4];
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (r < M && lane < KCH / 8) xst[r] = bld16(rx, (uint32_t)(r * (uint32_t)K + k0 + 8 * lane) * 2);
    scale_t<WDT> sv[NSTEP];
    u32x4_t wr[NSTEP];
#pragma unroll
    for (int c = 0; c < NSTEP; c++) {
      const uint32_t kk = k0 + c * KSTEP + EPL * g;
      sv[c] = scale_of<WDT>(rs, (uint32_t)nl * spr + (kk >> gs));
    }
#pragma unroll
    for (int c = 0; c < NSTEP; c++) {
      const uint32_t kk = k0 + c * KSTEP + EPL * g;
      wr[c] = bld16(rw, (uint32_t)nl * rowbytes + kk * BPE2 / 2);
    }
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (r < M && lane < KCH / 8) *reinterpret_cast<u32x4_t*>(xw + (r * KCH + 8 * lane) * 2) = xst[r];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int c = 0; c < NSTEP; c++) {
      bf16x8_t xa[MF];
#pragma unroll
      for (int j = 0; j < MF; j++) {
        const uint32_t kl = c * KSTEP + EPL * g + 8 * j;       // k within the chunk
        const uint32_t off = nl < M ? (nl * KCH + kl) * 2 : 4 * KCH * 2;
        xa[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(xw + off));
      }
      bf16x8_t b[4];
      dequant16<WDT>(wr[c], sv[c], b);
#pragma unroll
      for (int j = 0; j < MF; j++) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], b[j], acc, 0, 0, 0);
    }
    // the next chunk's staging overwrites this wave's region
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // acc[i] holds C[m = 4g + i][n = nl].
#pragma unroll
  for (int i = 0; i < 4; i++) red[(wave * 16 + 4 * g + i) * 16 + nl] = acc[i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 256; idx += blockDim.x) {
    const int m = idx >> 4, n = idx & 15;
    const int64_t col = n0 + n;
    if (m >= M || col >= N) continue;
    float s = 0.0f;
    for (int wv = 0; wv < S; wv++) s += red[(wv * 16 + m) * 16 + n];
    s *= WDT == W_FP8 ? chscale[col] * alpha : alpha;
    y[(int64_t)m * N + col] = (uint16_t)f32_to_bf16_bits(s);
  }
}

// 4 < M <= 16, TN (one or two) 16-column tiles per workgroup: each chunk's x
// rows are fetched whole (consecutive lanes read consecutive 16-byte pieces of a row)
// and pass through the wave's LDS region, piece p of row r at p ^ (r & 15), so
// that the 16 rows of one fragment read sit in distinct banks.  Read straight
// into the MFMA layout instead, a lane's four pieces of a row lie 64 bytes
// apart and each load touches two cache lines per row for one quarter of
// their bytes.  The next chunk's x, scales and weights are in flight while the
// current one is multiplied (two register sets, used in turn; a set past the
// wave's last chunk, and an x row past M, load from an offset outside the
// buffer range, which returns zeros without a memory access, so every load is
// issued unconditionally and the wait counts stay fixed).
template <int WDT, int NSTEP, int TN, int MG>
__global__ __launch_bounds__(TN * MG >= 4 ? 512 : 1024) void k_gemv_x16(const uint16_t* __restrict__ x, int M, int64_t N, int64_t K,
                                                  const uint8_t* __restrict__ w, const void* __restrict__ sc,
                                                  int group_shift, const float* __restrict__ chscale, float alpha,
                                                  uint16_t* __restrict__ y, int nchunk) {
  constexpr int EPL = WTraits<WDT>::bits == 4 ? 32 : 16;   // elements per lane per step
  constexpr int KSTEP = 4 * EPL;                            // K covered by a wave per step
  constexpr int KCH = NSTEP * KSTEP;                        // K per wave per chunk
  constexpr int MF = EPL / 8;                               // MFMAs per step
  constexpr int BPE2 = WTraits<WDT>::bits == 4 ? 1 : 2;     // bytes per 2 elements
  constexpr int SB = scale_bytes<WDT>();
  constexpr int XCH = KCH / 8;                              // 16-byte pieces per x row of a chunk
  constexpr int XL = 16 * MG * XCH / 64;                    // x loads per lane per chunk
  constexpr int XRB = KCH * 2;                              // bytes per x row of a chunk
  constexpr int XWB = 16 * MG * XRB;                        // per-wave x region
  static_assert(XCH % 16 == 0 && XCH <= 64, "x pieces are swizzled in groups of 16");
  static_assert(TN * MG * 1024 <= XWB, "the partial sums reuse the wave's x region");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int S = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * TN;
  const uint32_t rowbytes = (uint32_t)(K * BPE2 / 2);
  const int64_t nrows = N - n0 < 16 * TN ? N - n0 : 16 * TN;
  const int gs = gshift_of<WDT>(group_shift);
  const uint32_t spr = (uint32_t)(K >> gs);
  const auto rw = make_rsrc(w + n0 * rowbytes, nrows * rowbytes);
  const auto rs = make_rsrc(reinterpret_cast<const uint8_t*>(sc) + (WDT == W_FP8 ? 0 : n0 * spr * SB),
                            WDT == W_FP8 ? 0 : nrows * spr * SB);
  const auto rx = make_rsrc(x, (int64_t)M * K * 2);
  const int c0 = (int)((int64_t)wave * nchunk / S), niter = (int)((int64_t)(wave + 1) * nchunk / S) - c0;
  constexpr uint32_t OUT = 0x7FFFFFF0u;                     // past every range (all <= this many bytes)
  constexpr uint32_t SOUT = OUT / 4;                        // scale index past every scale range
  uint8_t* xw = smem + wave * XWB;

  struct Chunk {
    u32x4_t xs[XL];
    u32x4_t wr[NSTEP][TN];
    uint32_t sv[NSTEP][TN];                                 // raw bits, converted at the use
  };
  auto issue = [&](Chunk& b, int it) {
    const bool ok = it < niter;
    const uint32_t k0 = (uint32_t)((c0 + it) * KCH);
#pragma unroll
    for (int i = 0; i < XL; i++) {
      const int f = 64 * i + lane, r = f / XCH, p = f % XCH;
      b.xs[i] = bld16(rx, ok && r < M ? (uint32_t)(r * (uint32_t)K + k0 + 8 * p) * 2 : OUT);
    }
#pragma unroll
    for (int c = 0; c < NSTEP; c++)
#pragma unroll
      for (int t = 0; t < TN; t++) {
        const uint32_t kk = k0 + c * KSTEP + EPL * g;
        b.sv[c][t] = scale_raw_of<WDT>(rs, ok ? (uint32_t)(16 * t + nl) * spr + (kk >> gs) : SOUT);
      }
#pragma unroll
    for (int c = 0; c < NSTEP; c++)
#pragma unroll
      for (int t = 0; t < TN; t++) {
        const uint32_t kk = k0 + c * KSTEP + EPL * g;
        b.wr[c][t] = bld16(rw, ok ? (uint32_t)(16 * t + nl) * rowbytes + kk * BPE2 / 2 : OUT);
      }
  };
  f32x4_t acc[MG][TN];
#pragma unroll
  for (int q = 0; q < MG; q++)
#pragma unroll
    for (int t = 0; t < TN; t++) acc[q][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](Chunk& b) {
    // the previous chunk's fragment reads of the region come first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < XL; i++) {
      const int f = 64 * i + lane, r = f / XCH, p = f % XCH;
      if (r < M) *reinterpret_cast<u32x4_t*>(xw + r * XRB + ((p ^ (r & 15)) << 4)) = b.xs[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int c = 0; c < NSTEP; c++) {
      bf16x8_t xa[MG][MF];
#pragma unroll
      for (int q = 0; q < MG; q++) {
        const int row = 16 * q + nl, xr = row < M ? row : 0;  // rows past M read row 0; dropped
#pragma unroll
        for (int j = 0; j < MF; j++) {
          const int p = (c * KSTEP + EPL * g + 8 * j) >> 3;
          xa[q][j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(xw + xr * XRB + ((p ^ (xr & 15)) << 4)));
        }
      }
#pragma unroll
      for (int t = 0; t < TN; t++) {
        bf16x8_t bq[4];
        dequant16<WDT>(b.wr[c][t], scale_from_raw<WDT>(b.sv[c][t]), bq);
#pragma unroll
        for (int q = 0; q < MG; q++)
#pragma unroll
          for (int j = 0; j < MF; j++)
            acc[q][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q][j], bq[j], acc[q][t], 0, 0, 0);
      }
    }
  };
  Chunk ca, cb;
  issue(ca, 0);
  for (int it = 0; it < niter; it += 2) {
    issue(cb, it + 1);
    consume(ca);
    issue(ca, it + 2);
    if (it + 1 < niter) consume(cb);
  }

  // acc[q][t][i] holds C[m = 16q + 4g + i][n = nl] of tile t; the partial
  // sums go to the front of the wave's own x region once its reads are done
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* red = reinterpret_cast<float*>(xw);
#pragma unroll
  for (int q = 0; q < MG; q++)
#pragma unroll
    for (int t = 0; t < TN; t++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[((q * TN + t) * 16 + 4 * g + i) * 16 + nl] = acc[q][t][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MG * TN * 256; idx += blockDim.x) {
    const int qt = idx >> 8, q = qt / TN, t = qt % TN, m = 16 * q + ((idx >> 4) & 15), n = idx & 15;
    const int64_t col = n0 + 16 * t + n;
    if (m >= M || col >= N) continue;
    float s = 0.0f;
    for (int wv = 0; wv < S; wv++) s += reinterpret_cast<const float*>(smem + wv * XWB)[idx];
    s *= WDT == W_FP8 ? chscale[col] * alpha : alpha;
    y[(int64_t)m * N + col] = (uint16_t)f32_to_bf16_bits(s);
  }
}

// ---------------------------------------------------------------------------
// Prefill GEMM, 8-wave form
// ---------------------------------------------------------------------------
// 256x256 output tile per workgroup of 8 waves (8 along N, each 256x32, for
// 4-bit weights; 2 along M x 4 along N, each 128x64, for E4M3), MFMA 32x32x16
// bf16, K step 64, three LDS stages (four were
// measured no faster for 4-bit weights).  Two waves share
// each SIMD, so one wave's MFMAs overlap the other's dequantization and LDS
// reads.  Tiles arrive by direct-to-LDS buffer loads issued NSTAGE - 1 K steps
// ahead; one barrier per step both publishes a step's tiles and retires the
// reads of the stage the next loads overwrite.  x rows are 128 bytes in LDS with
// their 16-byte chunks XOR-swizzled by row (chunk c of row r sits at
// c ^ ((r >> 1) & 7)); W rows are swizzled at their 16-byte chunk granularity.
// Both placements were measured on gfx950 to read their fragments (32 rows x 2
// chunks) without LDS bank conflicts; c ^ (r & 7) takes about 1.7 times as long.
// Rows past M or N read as zeros through the buffer range; their results are
// not stored.
template <int WDT>
struct Gemm8 {
  static constexpr int BM = 256, BN = 256, BK = 64;
  // waves along N (the rest along M) and each wave's 32x32 MFMA tiles.  With
  // all 8 waves along N (4-bit weights) every W fragment is converted once per
  // workgroup instead of once per M-half, at twice the x fragment reads from
  // LDS: measured 8 % faster for INT4, 2 % for MXFP4, and 5 % slower for E4M3,
  // whose conversion is cheap and whose W tile is twice as large.
  static constexpr int NW = 8;                                  // waves per workgroup
  static constexpr int WN = WTraits<WDT>::bits == 4 ? 8 : 4;
  static constexpr int WM = NW / WN;
  static constexpr int TM = BM / WM, TN = BN / WN;            // rows and columns per wave
  static constexpr int MI = TM / 32, NJ = TN / 32;
  static constexpr int NSTAGE = 3;                              // loads run NSTAGE - 1 steps ahead
  // convert W one k16 slice ahead (4-bit weights: measured 1.5-2 % faster)
  // or one whole step ahead (8-bit weights: 10 % faster)
  static constexpr bool SLICE_AHEAD = WTraits<WDT>::bits == 4;
  static constexpr int wbytes = BK * WTraits<WDT>::bits / 8;   // packed bytes per W row per step
  static constexpr int A_TILE = BM * BK * 2;                    // 32 KB
  static constexpr int B_TILE = BN * wbytes;                    // 8 KB (4-bit) or 16 KB (8-bit)
  static constexpr int STAGE = A_TILE + B_TILE;
  static constexpr int LDS = NSTAGE * STAGE;
  static constexpr int A_DMA = A_TILE / 1024 / NW;              // 1 KB DMA instructions per wave
  static constexpr int B_DMA = B_TILE / 1024 / NW;
  static constexpr int LPR = wbytes / 16;                       // 16-byte chunks per W row
  // vector-memory instructions one step issues per lane: tile DMAs, scale loads
  static constexpr int VM_T = A_DMA + B_DMA;
  static constexpr int VM_S = WTraits<WDT>::bits == 4 ? 2 : 0;
};
// x rows (128 bytes): chunk c of row r sits at c ^ aswz(r).
__device__ __forceinline__ int aswz(int r) { return (r >> 1) & 7; }
// W rows of 32 or 64 bytes: chunk c of row r sits at c ^ bswz(r).
template <int LPR>
__device__ __forceinline__ int bswz(int r) { return LPR == 2 ? (r >> 3) & 1 : (r >> 1) & 3; }

template <int WDT>
__global__ __launch_bounds__(64 * Gemm8<WDT>::NW) void k_gemm8(const uint16_t* __restrict__ x, int64_t M, int64_t N, int64_t K,
                                              const uint8_t* __restrict__ w, const void* __restrict__ sc,
                                              int group_shift, const float* __restrict__ chscale, float alpha,
                                              uint16_t* __restrict__ y, int tiles_m, int tiles_n) {
  using C = Gemm8<WDT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / C::WN, wn = wave % C::WN;
  constexpr int MI = C::MI, NJ = C::NJ;
  const int l32 = lane & 31, h = lane >> 5;

  // XCD-aware order: consecutive workgroup ids land on different XCDs, so give
  // each XCD a contiguous range of tiles (m-major, which shares W panels).
  const int nwg = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if (nwg % 8 == 0) pid = (pid % 8) * (nwg / 8) + pid / 8;
  const int tn = pid % tiles_n, tm = pid / tiles_n;
  const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
  const int64_t rowbytes = K * WTraits<WDT>::bits / 8;
  const int64_t mrows = M - m0 < C::BM ? M - m0 : C::BM;
  const int64_t nrows = N - n0 < C::BN ? N - n0 : C::BN;
  const auto ra = make_rsrc(x + m0 * K, mrows * K * 2);
  const auto rb = make_rsrc(w + n0 * rowbytes, nrows * rowbytes);

  // DMA assignments.  A: 32 KB per stage = A_DMA instructions per wave, each 8 rows.
  uint32_t a_off[C::A_DMA];
#pragma unroll
  for (int i = 0; i < C::A_DMA; i++) {
    const int r = 8 * (wave * C::A_DMA + i) + (lane >> 3);
    const int c = (lane & 7) ^ aswz(r);
    a_off[i] = (uint32_t)r * (uint32_t)(K * 2) + 16 * c;
  }
  // B: rows of wbytes, lanes in row order, chunks swizzled by row.
  constexpr int LPR = C::LPR;
  uint32_t b_off[C::B_DMA];
#pragma unroll
  for (int i = 0; i < C::B_DMA; i++) {
    const int r = (1024 / C::wbytes) * (wave * C::B_DMA + i) + lane / LPR;
    b_off[i] = (uint32_t)(r * rowbytes) + 16 * ((lane % LPR) ^ bswz<LPR>(r));
  }
  auto issue = [&](int stage, int64_t k0) {
    uint8_t* A = lds + stage * C::STAGE;
    uint8_t* B = A + C::A_TILE;
#pragma unroll
    for (int i = 0; i < C::A_DMA; i++) lds_dma16(ra, A + (wave * C::A_DMA + i) * 1024, a_off[i] + (uint32_t)(k0 * 2));
#pragma unroll
    for (int i = 0; i < C::B_DMA; i++)
      lds_dma16(rb, B + (wave * C::B_DMA + i) * 1024, b_off[i] + (uint32_t)(k0 * WTraits<WDT>::bits / 8));
  };

  // scale rows of this lane's two 32-column subtiles (clamped; unused past N)
  int64_t srow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const int64_t n = n0 + wn * C::TN + 32 * j + l32;
    srow[j] = n < N ? n : N - 1;
  }
  // Scales are prefetched one step ahead as raw bits and converted only after
  // the next step's wait: converting at the load would make the wave wait for
  // the tile loads issued just before it.
  const int gs = gshift_of<WDT>(group_shift);
  auto scale_raw = [&](int j, int64_t k0) -> uint32_t {
    const int64_t kk = (k0 + 32 * h) >> gs;
    if constexpr (WDT == W_INT4) {
      return reinterpret_cast<const uint16_t*>(sc)[srow[j] * (K >> gs) + kk];
    } else if constexpr (WDT == W_FP4) {
      return reinterpret_cast<const uint8_t*>(sc)[srow[j] * (K >> 5) + kk];
    } else if constexpr (WDT == W_NV4) {
      // the two blocks of the lane's 32 elements: an even byte offset
      return *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(sc) + srow[j] * (K >> 4) + kk);
    } else if constexpr (WDT == W_UINT4) {
      return reinterpret_cast<const uint32_t*>(sc)[srow[j] * (K >> gs) + kk];
    } else {
      return 0u;
    }
  };
  auto scale_val = [](uint32_t raw) -> scale_t<WDT> { return scale_from_raw<WDT>(raw); };

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; i++)
#pragma unroll
    for (int j = 0; j < NJ; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  // Software pipeline.  Group k (step k's tiles) goes to stage k % NSTAGE,
  // issued at the top of step k - NSTAGE + 1; the scales of group k are loaded
  // at the top of step k - 2.  Step k runs four k16 slices of MFMAs on A from
  // LDS; while slice s runs, the W fragments of slice s + 1 are converted in
  // registers (during slice 3, those of slice 0 of step k + 1, from the next
  // stage), and the x fragments of slice s + 1 are read, so dequantization and
  // LDS reads overlap the matrix work and only two slices of converted W are
  // live.  The wait and barrier at the end of step k publish group k + 2 and
  // retire every read of stage k % NSTAGE, which step k + 1 refills.  The loop
  // is unrolled by two with ping-pong registers (no register copies).
  constexpr int NST = C::NSTAGE;
  static_assert(NST == 3 || NST == 4, "two or three steps of prefetch");
  const int nk = (int)(K / C::BK);
  uint32_t sa[NJ], sb[NJ] = {};
  // issue order: t0 s0 t1 [t2] s1, so that step 0's closing wait sees the
  // same queue as every later step's
  issue(0, 0);
#pragma unroll
  for (int j = 0; j < NJ; j++) sa[j] = scale_raw(j, 0);
  if (nk > 1) issue(1, C::BK);
  if (NST == 4 && nk > 2) issue(2, 2 * C::BK);
  if (nk > 1) {
#pragma unroll
    for (int j = 0; j < NJ; j++) sb[j] = scale_raw(j, C::BK);
  }
  wait_vm<0>();
  tile_barrier();

  // 4-bit W: the lane's 16-byte chunk of each column subtile, read once per
  // step (one 16-byte LDS read instead of four 4-byte ones)
  auto wchunk = [&](const uint8_t* B, u32x4_t (&wc)[NJ]) {
    if constexpr (WTraits<WDT>::bits == 4) {
#pragma unroll
      for (int j = 0; j < NJ; j++) {
        const int br = wn * C::TN + 32 * j + l32;
        wc[j] = ld16(B + br * C::wbytes + 16 * (h ^ bswz<LPR>(br)));
      }
    }
  };
  // quarter q (k16 slice q) of a step's W fragments for both column subtiles
  auto dequant_q = [&](const uint8_t* B, const u32x4_t (&wc)[NJ], int q, const scale_t<WDT> (&cs)[NJ],
                       bf16x8_t (&out)[4][NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int br = wn * C::TN + 32 * j + l32;
      const uint8_t* bp = B + br * C::wbytes;
      const int sw = bswz<LPR>(br);
      if constexpr (WTraits<WDT>::bits == 4) {
        const uint32_t wd = wc[j][q];
        uint32_t o[4];
        if constexpr (WDT == W_INT4) dq_int4_word(wd, cs[j], o);
        else if constexpr (WDT == W_NV4) dq_nv4_word(wd, q < 2 ? cs[j].lo : cs[j].hi, o);
        else if constexpr (WDT == W_UINT4) dq_uint4_word(wd, cs[j].s, cs[j].b, o);
        else dq_fp4_word(wd, cs[j], o);
        out[q][j] = as_bf16x8(o[0], o[1], o[2], o[3]);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(bp + 16 * ((2 * h + (q >> 1)) ^ sw) + 8 * (q & 1));
        out[q][j] = as_bf16x8(dq_fp8_pair<false>(v.x), dq_fp8_pair<true>(v.x), dq_fp8_pair<false>(v.y),
                              dq_fp8_pair<true>(v.y));
      }
    }
  };
  if constexpr (C::SLICE_AHEAD) {
  // Slice-ahead pipeline: the W fragments of k16 slice s + 1 are converted
  // while slice s runs its MFMAs (slice 0 of step kt + 1 during slice 3 of
  // step kt), so only two slices of B fragments are live.
  bf16x8_t bsl[2][NJ];
  u32x4_t wca[NJ], wcb[NJ];
  scale_t<WDT> cca[NJ], ccb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; j++) cca[j] = scale_val(sa[j]);
  wchunk(lds + C::A_TILE, wca);
  {
    bf16x8_t tmp[4][NJ];
    dequant_q(lds + C::A_TILE, wca, 0, cca, tmp);
#pragma unroll
    for (int j = 0; j < NJ; j++) bsl[0][j] = tmp[0][j];
  }
  int stage = 0;
  auto step = [&](int kt, u32x4_t (&wcur)[NJ], scale_t<WDT> (&ccur)[NJ], u32x4_t (&wnext)[NJ],
                  scale_t<WDT> (&cnext)[NJ], uint32_t (&snext)[NJ], uint32_t (&sload)[NJ]) {
    const int st1 = stage == NST - 1 ? 0 : stage + 1;
    const int stl = stage == 0 ? NST - 1 : stage - 1;
#pragma unroll
    for (int j = 0; j < NJ; j++) cnext[j] = scale_val(snext[j]);
    if (kt + NST - 1 < nk) issue(stl, (int64_t)(kt + NST - 1) * C::BK);
    if (kt + 2 < nk) {
#pragma unroll
      for (int j = 0; j < NJ; j++) sload[j] = scale_raw(j, (int64_t)(kt + 2) * C::BK);
    }
    const uint8_t* A = lds + stage * C::STAGE;
    const uint8_t* Bc = A + C::A_TILE;
    const uint8_t* Bn = lds + st1 * C::STAGE + C::A_TILE;
    wchunk(Bn, wnext);
    auto load_a = [&](int s4, bf16x8_t (&dst)[MI]) {
#pragma unroll
      for (int i = 0; i < MI; i++) {
        const int r = wm * C::TM + 32 * i + l32;
        dst[i] = as_bf16x8(ld16(A + r * 128 + (((4 * h + s4) ^ aswz(r)) << 4)));
      }
    };
    bf16x8_t af[2][MI];
    load_a(0, af[0]);
#pragma unroll
    for (int s4 = 0; s4 < 4; s4++) {
      if (s4 < 3) load_a(s4 + 1, af[(s4 + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      {
        bf16x8_t tmp[4][NJ];
        if (s4 < 3) dequant_q(Bc, wcur, s4 + 1, ccur, tmp);
        else dequant_q(Bn, wnext, 0, cnext, tmp);
        const int q = s4 < 3 ? s4 + 1 : 0;
#pragma unroll
        for (int j = 0; j < NJ; j++) bsl[(s4 + 1) & 1][j] = tmp[q][j];
      }
#pragma unroll
      for (int i = 0; i < MI; i++)
#pragma unroll
        for (int j = 0; j < NJ; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s4 & 1][i], bsl[s4 & 1][j], acc[i][j], 0, 0, 0);
    }
    if constexpr (NST == 4) {
      if (kt + 3 < nk) wait_vm<C::VM_T + 2 * C::VM_S>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    tile_barrier();
    stage = st1;
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, wca, cca, wcb, ccb, sb, sa);
    if (kt + 1 < nk) step(kt + 1, wcb, ccb, wca, cca, sa, sb);
  }
  } else {
  // Step-ahead form (8-bit weights, whose 2 x 4 waves convert from LDS per
  // slice): step k converts all of step k + 1's W fragments.
  bf16x8_t ba[4][NJ], bb[4][NJ];
  {
    scale_t<WDT> c0[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) c0[j] = scale_val(sa[j]);
    u32x4_t wc[NJ];
    wchunk(lds + C::A_TILE, wc);
#pragma unroll
    for (int q = 0; q < 4; q++) dequant_q(lds + C::A_TILE, wc, q, c0, ba);
  }

  int stage = 0;
  auto step = [&](int kt, bf16x8_t (&bcur)[4][NJ], bf16x8_t (&bnext)[4][NJ], uint32_t (&snext)[NJ],
                  uint32_t (&sload)[NJ]) {
    const int st1 = stage == NST - 1 ? 0 : stage + 1;
    const int stl = stage == 0 ? NST - 1 : stage - 1;        // stage of group kt + NST - 1
    scale_t<WDT> cn[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) cn[j] = scale_val(snext[j]);
    if (kt + NST - 1 < nk) issue(stl, (int64_t)(kt + NST - 1) * C::BK);
    if (kt + 2 < nk) {
#pragma unroll
      for (int j = 0; j < NJ; j++) sload[j] = scale_raw(j, (int64_t)(kt + 2) * C::BK);
    }
    const uint8_t* A = lds + stage * C::STAGE;
    const uint8_t* Bn = lds + st1 * C::STAGE + C::A_TILE;
    u32x4_t wc[NJ];
    wchunk(Bn, wc);
    auto load_a = [&](int s4, bf16x8_t (&dst)[MI]) {
#pragma unroll
      for (int i = 0; i < MI; i++) {
        const int r = wm * C::TM + 32 * i + l32;
        dst[i] = as_bf16x8(ld16(A + r * 128 + (((4 * h + s4) ^ aswz(r)) << 4)));
      }
    };
    // PF: the x fragments of slice s4 + 1 are read during slice s4
    constexpr bool PF = C::WN == 8;
    bf16x8_t af[PF ? 2 : 1][MI];
    if constexpr (PF) load_a(0, af[0]);
#pragma unroll
    for (int s4 = 0; s4 < 4; s4++) {
      if constexpr (PF) {
        if (s4 < 3) load_a(s4 + 1, af[(s4 + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        load_a(s4, af[0]);
      }
      const int cur = PF ? (s4 & 1) : 0;
      dequant_q(Bn, wc, s4, cn, bnext);
#pragma unroll
      for (int i = 0; i < MI; i++)
#pragma unroll
        for (int j = 0; j < NJ; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bcur[s4][j], acc[i][j], 0, 0, 0);
    }
    // group kt + 2 complete: with four stages the loads queued behind it are
    // the scales of group kt + 1, group kt + 3 and the scales of group kt + 2
    if constexpr (NST == 4) {
      if (kt + 3 < nk) wait_vm<C::VM_T + 2 * C::VM_S>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    tile_barrier();
    stage = st1;
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, ba, bb, sb, sa);
    if (kt + 1 < nk) step(kt + 1, bb, ba, sa, sb);
  }

  }
  // epilogue: C element r of a 32x32 tile sits at row 8*(r/4) + 4*h + r%4, col l32.
  // Stores go through a buffer range covering the tile's rows below M, so the
  // rest are dropped by the hardware and offsets stay 32-bit.
  const auto ry = make_rsrc(y + m0 * N, mrows * N * 2);
  const uint32_t rowb = (uint32_t)(N * 2);
  float cs[NJ];
  uint32_t cb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const int64_t col = n0 + wn * C::TN + 32 * j + l32;
    cs[j] = alpha;
    if constexpr (WDT == W_FP8) cs[j] = col < N ? chscale[col] * alpha : 0.0f;
    cb[j] = col < N ? (uint32_t)(col * 2) : 0x80000000u;    // columns past N: out of range
  }
#pragma unroll
  for (int i = 0; i < MI; i++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const uint32_t lr = (uint32_t)(wm * C::TM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3));
      const uint32_t off = lr * rowb;
#pragma unroll
      for (int j = 0; j < NJ; j += 2) {
        const int j1 = j + 1 < NJ ? j + 1 : j;                 // the pair's second column subtile
        const uint32_t pr = pack_bf16x2(acc[i][j][r] * cs[j], acc[i][j1][r] * cs[j1]);
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pr & 0xFFFFu), ry, (int)(off + cb[j]), 0, 0);
        if (j1 != j) __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pr >> 16), ry, (int)(off + cb[j1]), 0, 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode GEMV, LDS-ring form (M <= 4)
// ---------------------------------------------------------------------------
// A workgroup of 4 waves owns 16 output columns (or 8 over both halves of K,
// see gemv_ring_tile); wave w owns the K-slice of SPW steps
// [w*SPW, (w+1)*SPW).  Packed weights never occupy VGPRs while in
// flight: each step's 16 rows x 64 bytes (1 KB) are fetched by direct-to-LDS
// buffer loads R steps ahead into a ring of R + 1 slots of the wave, so many
// steps of every wave are outstanding at once; the extra slot lets each step
// refill the slot the previous step read.  Lane l fetches, and later reads back, the 16
// bytes it feeds to the MFMA (row l % 16, K offset 32 or 16 elements times
// l / 16), so the LDS ring needs no cross-lane synchronisation.  The x rows of
// the slice are fetched the same way once.  MFMA rows >= M read row 0 of x;
// those output rows are discarded.

// Kernels that may take more than 64 KB of dynamic LDS raise their limit to the
// CU's 160 KB once per device before their first launch there.
template <auto KERNEL>
hipError_t allow_lds(size_t bytes) {
  static bool done[64] = {};
  if (bytes <= 65536) return hipSuccess;
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && done[dev]) return hipSuccess;
  const hipError_t f =
      hipFuncSetAttribute(reinterpret_cast<const void*>(KERNEL), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (f == hipSuccess && dev >= 0 && dev < 64) done[dev] = true;
  return f;
}

// Compute units of the current device, queried once per device.
hipError_t cu_count(int* n) {
  static int cached[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) {
    *n = cached[dev];
    return hipSuccess;
  }
  e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*n <= 0) *n = 1;
  if (dev >= 0 && dev < 64) cached[dev] = *n;
  return hipSuccess;
}

// Ring slots of the LDS ring: one more than the prefetch depth R, so that a
// refill never targets the slot the current step reads.
__host__ __device__ constexpr int ring_slots(int spw, int r) { return r < spw ? r + 1 : r; }

// E4M3 weights bypass the LDS ring: every step of the slice is loaded into
// registers up front (measured faster for 1-3 tokens, where the conversion is
// cheap; for INT4 the conversions then bunch behind the last arrivals and the
// ring is faster).
template <int WDT>
__host__ __device__ constexpr bool ring_regw(bool xs) {
  return WDT == W_FP8 && !xs;
}

// Per-wave LDS of a ring tile (bytes): the ring, the x rows (the whole slice,
// or with XS a 4-token x chunk in every slot) and the slice's scales.
template <int WDT, int GSH>
__host__ __device__ constexpr int ring_wave_bytes(int spwe, int r, bool half, bool xs, int m) {
  const int kstep = WTraits<WDT>::bits == 4 ? 128 : 64;
  const int ksl = spwe * kstep;
  const int xr = half ? 2 : 1;
  const int sbrow = (ksl >> gshift_of<WDT>(GSH)) * scale_bytes<WDT>();
  const int sbytes = WDT == W_FP8 ? 0 : 16 * (sbrow < 16 ? 16 : (sbrow + 15) / 16 * 16);
  const int ns = ring_slots(spwe, r);
  const int ring = xs ? ns * (1024 + xr * 4 * kstep * 2) : (ring_regw<WDT>(xs) ? 0 : ns * 1024) + xr * m * ksl * 2;
  return ring + ((sbytes + 15) & ~15);
}

// Prefetch depth of the 8-column tiles (their slices are half as long; with
// XS at most 2, which keeps their larger slots within the 16-column tiles' LDS)
__host__ __device__ constexpr int ring_half_depth(int spw, int r, bool xs) {
  const int sph = spw / 2;
  const int rh = r < sph ? r : sph;
  return xs && rh > 2 ? 2 : rh;
}

// s_waitcnt vmcnt(n) for an n the caller knows at compile time after
// unrolling (folds to one instruction)
template <int C = 0>
__device__ __forceinline__ void wait_vm_n(int n) {
  if constexpr (C < 40) {
    if (n == C) wait_vm<C>();
    else wait_vm_n<C + 1>(n);
  } else {
    wait_vm<0>();
  }
}

// One wave's part of a ring tile.  HALF = false: the tile is 16 columns of W
// over all of K, wave w owns steps [w*SPWE, (w+1)*SPWE) of K.  HALF = true: the
// tile is 8 columns, and the MFMA's 16 columns are those 8 columns over the two
// halves of K (MFMA column v: W column v % 8, K half v / 8); the MFMA's rows
// 0..7 carry the tokens over the first half of K and rows 8..15 over the
// second, so C[m][v] (v < 8) and C[8 + m][8 + v] are the two halves' partial
// sums and the other two quadrants are discarded.  Wave w owns steps
// [w*SPWE, (w+1)*SPWE) of each K half.  Needs M <= 8.
// XS: the x rows travel with the weights, a chunk of up to 4 tokens in every
// ring slot, instead of the whole slice up front (less LDS at M = 4, so that
// four workgroups fit on a CU).  Needs M <= 4.
template <int WDT, int SPWE, int R, int NW, int GSH, bool HALF, bool XS>
__device__ __forceinline__ void gemv_ring_tile(const uint16_t* __restrict__ x, int M, int64_t N, int64_t K,
                                               const uint8_t* __restrict__ w, const void* __restrict__ sc,
                                               const float* __restrict__ chscale, float alpha,
                                               uint16_t* __restrict__ y, int64_t n0, uint8_t* smem) {
  constexpr int EPL = WTraits<WDT>::bits == 4 ? 32 : 16;
  constexpr int KSTEP = 4 * EPL;
  constexpr int KSL = SPWE * KSTEP;                           // K of one wave's slice (per half)
  constexpr int MF = EPL / 8;
  constexpr int BPE2 = WTraits<WDT>::bits == 4 ? 1 : 2;
  constexpr int XROW = KSL * 2;                               // bytes of one x row of the slice
  constexpr int NR = HALF ? 8 : 16;                           // W rows of the tile
  static_assert(R <= SPWE, "ring larger than the slice");
  constexpr int NS = ring_slots(SPWE, R);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, g = lane >> 4;
  // MFMA column nl: W row wr of the tile, K half hp (the same split for the
  // MFMA row nl of the x operand)
  const int wr = HALF ? (nl & 7) : nl, hp = HALF ? nl >> 3 : 0;
  const uint32_t rowbytes = (uint32_t)(K * BPE2 / 2);
  const int64_t nrows = N - n0 < NR ? N - n0 : NR;
  constexpr int gs = gshift_of<WDT>(GSH);
  const uint32_t spr = (uint32_t)(K >> gs);                  // scales per row
  constexpr int SB = scale_bytes<WDT>();
  constexpr uint32_t sbrow = (uint32_t)(KSL >> gs) * SB;     // scale bytes per row of the slice
  const auto rw = make_rsrc(w + n0 * rowbytes, nrows * rowbytes);
  const auto rs = make_rsrc(reinterpret_cast<const uint8_t*>(sc) + (WDT == W_FP8 ? 0 : n0 * spr * SB),
                            WDT == W_FP8 ? 0 : nrows * spr * SB);
  const auto rx = make_rsrc(x, (int64_t)M * K * 2);
  const uint32_t khalf = HALF ? (uint32_t)(K / 2) : 0u;
  const uint32_t kbase = (uint32_t)(wave * KSL);             // within the K half
  // per-wave LDS: ring | x rows of the slice (HALF: M rows per K half) |
  // scales of the slice (16 MFMA columns, row stride srs).  With XS a slot
  // holds the step's 1 KB of weights, then 4 token rows of x per K half.
  constexpr int XR = HALF ? 2 : 1;
  constexpr uint32_t srs = sbrow < 16 ? 16 : (sbrow + 15) / 16 * 16;   // LDS row stride of the scales
  constexpr int XRB = KSTEP * 2;                              // bytes of one x row of a step
  constexpr int XCH = 4 * XRB;                                // x chunk of one K half
  constexpr int SLOT = XS ? 1024 + XR * XCH : 1024;
  constexpr int VMS = XS ? 1 + XR : 1;                        // loads per step
  const int wstride = ring_wave_bytes<WDT, GSH>(SPWE, R, HALF, XS, M);
  constexpr bool REGW = ring_regw<WDT>(XS);
  uint8_t* ring = smem + wave * wstride;
  uint8_t* xl = ring + (REGW ? 0 : NS * SLOT);
  uint8_t* sl = xl + (XS ? 0 : XR * M * XROW);

  // 1) scales of the slice.  When a row of the slice holds at least 16 bytes
  //    of scales, they arrive by DMA, 16 bytes per lane, the row's window
  //    rounded up to whole 16-byte pieces (the bytes past the slice are not
  //    used; past the buffer range they read as zeros); for thinner slices
  //    every lane loads its own per-step scales instead (a 16-byte window
  //    could leave the buffer range at the last row and read as zeros).
  constexpr bool sdma = sbrow >= 16;
  uint32_t svr[SPWE];
  if constexpr (WDT != W_FP8) {
    if constexpr (sdma) {
      // 16 MFMA columns x cpr chunks; one DMA instruction moves 64 of them (1 KB)
      constexpr int cpr = (int)srs / 16;
#pragma unroll
      for (int q = 0; q < (16 * cpr + 63) / 64; q++) {
        const int L = 64 * q + lane;
        const int v = L / cpr, vr = HALF ? (v & 7) : v, vh = HALF ? v >> 3 : 0;
        if (L < 16 * cpr)
          lds_dma16(rs, sl + 1024 * q,
                    (uint32_t)vr * spr * SB + ((vh * khalf + kbase) >> gs) * SB + 16 * (L % cpr));
      }
    } else {
#pragma unroll
      for (int c = 0; c < SPWE; c++)
        svr[c] = scale_raw_of<WDT>(rs, (uint32_t)wr * spr + ((hp * khalf + kbase + c * KSTEP + EPL * g) >> gs));
    }
  }
  // 2) x rows of the slice, 1 KB per DMA instruction (HALF: both K halves)
  if constexpr (!XS) {
#pragma unroll
    for (int h = 0; h < XR; h++)
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (r < M)
#pragma unroll
          for (int q = 0; q < (XROW + 1023) / 1024; q++)
            if (q * 1024 + lane * 16 < XROW)
              lds_dma16(rx, xl + (h * M + r) * XROW + q * 1024,
                        (uint32_t)(r * (uint32_t)K + h * khalf + kbase + q * 512 + 8 * lane) * 2);
  }
  // 3) the first R steps.  XS: lane L of a K half's x load moves 16 bytes of
  //    token L / (XRB / 16) (lanes of tokens >= M stay idle)
  const uint32_t wlane = (uint32_t)wr * rowbytes + (hp * khalf + kbase + EPL * g) * BPE2 / 2;
  constexpr int XCPR = XRB / 16;                              // 16-byte chunks per x row of a step
  const int xtok = lane / XCPR;
  const uint32_t xlane = (uint32_t)(xtok * (uint32_t)K + kbase + 8 * (lane % XCPR)) * 2;
  u32x4_t wreg[REGW ? SPWE : 1];
  auto issue_step = [&](int slot, int c) {
    uint8_t* sp = ring + slot * SLOT;
    if constexpr (REGW) wreg[c] = bld16(rw, wlane + c * KSTEP * BPE2 / 2);
    else lds_dma16(rw, sp, wlane, c * KSTEP * BPE2 / 2);
    if constexpr (XS) {
#pragma unroll
      for (int h = 0; h < XR; h++)
        if (xtok < M && lane < 4 * XCPR) lds_dma16(rx, sp + 1024 + h * XCH, xlane, (h * khalf + c * KSTEP) * 2);
    }
  };
#pragma unroll
  for (int c = 0; c < (REGW ? SPWE : R); c++) issue_step(c, c);

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int tok = HALF ? (nl & 7) : nl;                       // token of this lane's x operand row
  const int xtr = tok < M ? tok : 0;
  const uint8_t* xrow = XS ? ring + 1024 + hp * XCH + xtr * XRB : xl + (hp * M + xtr) * XROW;
  // FASTQ: the INT4 form without per-weight conversion (see below), chosen
  // once per wave for all of its steps
  auto run_steps = [&](auto fast_tag) {
    constexpr bool FASTQ = decltype(fast_tag)::value;
#pragma unroll
    for (int c = 0; c < SPWE; c++) {
      // step loads issued after step c's: min(R-1, SPWE-1-c) steps of VMS loads
      // (each step issues its refill after this wait)
      wait_vm_n(REGW ? SPWE - 1 - c : (c + R - 1 < SPWE ? R - 1 : SPWE - 1 - c) * VMS);
      if (!REGW && c + R < SPWE) {
        // step c + R goes to the slot step c - 1 read: that read returned before
        // step c - 1's conversion, and nothing may be scheduled across the
        // barrier (a DMA write is not ordered after an earlier LDS read)
        __builtin_amdgcn_sched_barrier(0);
        issue_step((c + R) % NS, c + R);
      }
      const u32x4_t wv = REGW ? wreg[c] : *reinterpret_cast<const u32x4_t*>(ring + (c % NS) * SLOT + lane * 16);
      scale_t<WDT> scv{};
      if constexpr (WDT == W_INT4) {
        const uint32_t gi = (uint32_t)(c * KSTEP + EPL * g) >> gs;
        scv = bf16_to_f32(sdma ? (uint32_t)*reinterpret_cast<const uint16_t*>(sl + nl * srs + 2 * gi) : svr[c]);
      } else if constexpr (WDT == W_FP4) {
        const uint32_t gi = (uint32_t)(c * KSTEP + EPL * g) >> 5;
        scv = sdma ? e8m0_as_scale(sl[nl * srs + gi]) : scale_from_raw<WDT>(svr[c]);
      } else if constexpr (WDT == W_NV4) {
        const uint32_t gi = (uint32_t)(c * KSTEP + EPL * g) >> 4;
        scv = scale_from_raw<WDT>(sdma ? (uint32_t)*reinterpret_cast<const uint16_t*>(sl + nl * srs + gi) : svr[c]);
      } else if constexpr (WDT == W_UINT4) {
        const uint32_t gi = (uint32_t)(c * KSTEP + EPL * g) >> gs;
        scv = scale_from_raw<WDT>(sdma ? *reinterpret_cast<const uint32_t*>(sl + nl * srs + 4 * gi) : svr[c]);
      }
      bf16x8_t xa[MF];
#pragma unroll
      for (int j = 0; j < MF; j++)
        xa[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
            xrow + (XS ? (c % NS) * SLOT + (EPL * g + 8 * j) * 2 : (c * KSTEP + EPL * g + 8 * j) * 2)));
      if constexpr (FASTQ) {
        if constexpr (WDT == W_INT4) mma_int4_exact_codes(xa, wv, scv, acc);
      } else {
        bf16x8_t b[4];
        dequant16<WDT>(wv, scv, b);
#pragma unroll
        for (int j = 0; j < MF; j++) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], b[j], acc, 0, 0, 0);
      }
    }
  };
  // INT4 groups of 128: a step covers one group per row.  When every scale of
  // the wave's slice has a 5-bit significand, every step takes the exact-code
  // form (mma_int4_exact_codes); otherwise every weight is converted to
  // bf16(q s).  The choice waits for the first step's loads (the scales were
  // issued before them), as the first step would.
  if constexpr (WDT == W_INT4 && gs == 7) {
    wait_vm_n(REGW ? SPWE - 1 : (R - 1 < SPWE ? R - 1 : SPWE - 1) * VMS);
    bool mine = true;
#pragma unroll
    for (int c = 0; c < SPWE; c++)
      mine &= int4_scale_short(sdma ? (uint32_t)*reinterpret_cast<const uint16_t*>(sl + nl * srs + 2 * c) : svr[c]);
    if (__builtin_amdgcn_ballot_w64(!mine) == 0) run_steps(std::true_type{});
    else run_steps(std::false_type{});
  } else {
    run_steps(std::false_type{});
  }

  // split-K reduction in the (consumed) front of the workgroup's LDS
  float* red = reinterpret_cast<float*>(smem);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; i++) red[(wave * 16 + 4 * g + i) * 16 + nl] = acc[i];
  __syncthreads();
  if (threadIdx.x < 16 * NR) {
    const int m = threadIdx.x / NR, n = threadIdx.x % NR;
    const int64_t col = n0 + n;
    if (m < M && col < N) {
      float s = 0.0f;
#pragma unroll
      for (int wv = 0; wv < NW; wv++) {
        s += red[(wv * 16 + m) * 16 + n];
        if constexpr (HALF) s += red[(wv * 16 + 8 + m) * 16 + 8 + n];
      }
      s *= WDT == W_FP8 ? chscale[col] * alpha : alpha;
      y[(int64_t)m * N + col] = (uint16_t)f32_to_bf16_bits(s);
    }
  }
}

// GSH: log2 of the INT4 scale group (a template parameter, so that every
// scale address is a compile-time offset).  Workgroups below nfull take
// 16-column tiles, the rest 8-column tiles from column 16 * nfull on: the
// host turns a last, partial round of tiles over the CUs into twice as many
// half tiles, so that every CU gets the same work.
template <int WDT, int SPW, int R, int NW, int GSH, bool XS>
__global__ __launch_bounds__(64 * NW) void k_gemv_ring(const uint16_t* __restrict__ x, int M, int64_t N, int64_t K,
                                                  const uint8_t* __restrict__ w, const void* __restrict__ sc,
                                                  const float* __restrict__ chscale, float alpha,
                                                  uint16_t* __restrict__ y, int nfull) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int b = (int)blockIdx.x;
  if constexpr (SPW >= 2) {
    constexpr int SPH = SPW / 2, RH = ring_half_depth(SPW, R, XS);
    if (b >= nfull) {
      gemv_ring_tile<WDT, SPH, RH, NW, GSH, true, XS>(x, M, N, K, w, sc, chscale, alpha, y,
                                                  (int64_t)nfull * 16 + (int64_t)(b - nfull) * 8, smem);
      return;
    }
  }
  gemv_ring_tile<WDT, SPW, R, NW, GSH, false, XS>(x, M, N, K, w, sc, chscale, alpha, y, (int64_t)b * 16, smem);
}

// Split of the K loop: T = K / KSTEP steps = nchunk chunks of NSTEP steps over
// S <= smax waves (the largest NSTEP dividing T; as many waves as there are
// chunks, up to smax, shares differing by at most one chunk).
struct GemvSplit { int nstep, S, nchunk; };
inline GemvSplit gemv_split(int64_t T, int maxstep, int smax) {
  int ns = maxstep;
  while (ns > 1 && T % ns) ns >>= 1;
  const int64_t chunks = T / ns;
  return GemvSplit{ns, (int)(chunks < smax ? chunks : smax), (int)chunks};
}

template <int WDT, int NSTEP>
hipError_t gemv_go(const GemvSplit& sp, const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w,
             const void* sc, int group, const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  const unsigned grid = (unsigned)((N + 15) / 16);
  constexpr int KCH = NSTEP * (WTraits<WDT>::bits == 4 ? 128 : 64);
  const size_t lds = (size_t)sp.S * (4 * KCH * 2 + 64) + (size_t)sp.S * 1024;
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;
  const hipError_t e = allow_lds<k_gemv<WDT, NSTEP>>(lds);
  if (e != hipSuccess) return e;
  k_gemv<WDT, NSTEP><<<grid, 64 * sp.S, lds, s>>>(x, (int)M, N, K, w, sc, gshift, ch, alpha, y, sp.nchunk);
  return hipSuccess;
}

template <int WDT>
hipError_t gemv_nstep(const GemvSplit& sp, const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                      const void* sc, int group, const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  switch (sp.nstep) {
    case 8: if constexpr (WTraits<WDT>::bits == 8) return gemv_go<WDT, 8>(sp, x, M, N, K, w, sc, group, ch, alpha, y, s);
            [[fallthrough]];
    case 4: return gemv_go<WDT, 4>(sp, x, M, N, K, w, sc, group, ch, alpha, y, s);
    case 2: return gemv_go<WDT, 2>(sp, x, M, N, K, w, sc, group, ch, alpha, y, s);
    default: return gemv_go<WDT, 1>(sp, x, M, N, K, w, sc, group, ch, alpha, y, s);
  }
}

template <int WDT, int NSTEP, int TN, int MG>
hipError_t x16_go(const GemvSplit& sp, const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                  const void* sc, int group, const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  const unsigned grid = (unsigned)((N + 16 * TN - 1) / (16 * TN));
  constexpr int KCH = NSTEP * (WTraits<WDT>::bits == 4 ? 128 : 64);
  const size_t lds = (size_t)sp.S * 16 * MG * KCH * 2;
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;
  const hipError_t e = allow_lds<k_gemv_x16<WDT, NSTEP, TN, MG>>(lds);
  if (e != hipSuccess) return e;
  k_gemv_x16<WDT, NSTEP, TN, MG><<<grid, 64 * sp.S, lds, s>>>(x, (int)M, N, K, w, sc, gshift, ch, alpha, y,
                                                             sp.nchunk);
  return hipSuccess;
}

// 4 < M <= 16: the 16 x rows of the wave's slice do not fit a wave's LDS
// share, so each step's x chunk (16 rows x 128 or 64 k) travels through its
// own ring next to the weights, fetched by direct-to-LDS loads (x is read from
// L2 by every workgroup).  A row's 16-byte chunks are XOR-swizzled by the row
// so that the 16 lanes reading one chunk of 16 rows use distinct banks; rows
// >= M read as zeros.  Scales come from per-lane loads issued up front.
template <int WDT, int SPW, int R, int NW, int CT, int GSH>
__global__ __launch_bounds__(64 * NW) void k_gemv_ring16(const uint16_t* __restrict__ x, int M, int64_t N,
                                                    int64_t K, const uint8_t* __restrict__ w,
                                                    const void* __restrict__ sc, const float* __restrict__ chscale,
                                                    float alpha, uint16_t* __restrict__ y) {
  constexpr int EPL = WTraits<WDT>::bits == 4 ? 32 : 16;
  constexpr int KSTEP = 4 * EPL;
  constexpr int KSL = SPW * KSTEP;
  constexpr int MF = EPL / 8;
  constexpr int BPE2 = WTraits<WDT>::bits == 4 ? 1 : 2;
  constexpr int XRB = KSTEP * 2;                              // bytes of one x row of a step
  constexpr int XSLOT = 16 * XRB;                             // 4 KB or 2 KB
  constexpr int XQ = XSLOT / 1024;                            // x DMA instructions per step
  constexpr int RPI = 1024 / XRB;                             // x rows per DMA instruction
  constexpr int CPR = XRB / 16;                               // 16-byte chunks per x row
  constexpr int VMS = CT + XQ;                                // loads per step per lane
  constexpr int SLOT = CT * 1024 + XSLOT;                     // CT weight chunks, then x
  static_assert(R <= SPW && R == 2, "two-deep ring");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * CT;
  const uint32_t rowbytes = (uint32_t)(K * BPE2 / 2);
  const int64_t nrows = N - n0 < 16 * CT ? N - n0 : 16 * CT;
  constexpr int gs = gshift_of<WDT>(GSH);
  const uint32_t spr = (uint32_t)(K >> gs);
  constexpr int SB = scale_bytes<WDT>();
  const auto rw = make_rsrc(w + n0 * rowbytes, nrows * rowbytes);
  const auto rs = make_rsrc(reinterpret_cast<const uint8_t*>(sc) + (WDT == W_FP8 ? 0 : n0 * spr * SB),
                            WDT == W_FP8 ? 0 : nrows * spr * SB);
  const auto rx = make_rsrc(x, (int64_t)M * K * 2);
  const uint32_t kbase = (uint32_t)(wave * KSL);
  uint8_t* ring = smem + wave * (R * SLOT);

  uint32_t svr[SPW][CT];
  if constexpr (WDT != W_FP8) {
#pragma unroll
    for (int c = 0; c < SPW; c++)
#pragma unroll
      for (int t = 0; t < CT; t++)
        svr[c][t] = scale_raw_of<WDT>(rs, (uint32_t)(16 * t + nl) * spr + ((kbase + c * KSTEP + EPL * g) >> gs));
  }
  const uint32_t wlane = (uint32_t)nl * rowbytes + (kbase + EPL * g) * BPE2 / 2;
  uint32_t xoff[XQ];
#pragma unroll
  for (int q = 0; q < XQ; q++) {
    const int r = q * RPI + lane / CPR;
    const int c = (lane % CPR) ^ (r & (CPR - 1));
    xoff[q] = (uint32_t)(r * (uint32_t)K + kbase + 8 * c) * 2;
  }
  auto issue = [&](int slot, int step) {
    uint8_t* b = ring + slot * SLOT;
#pragma unroll
    for (int t = 0; t < CT; t++) lds_dma16(rw, b + t * 1024, wlane + 16 * t * rowbytes + step * KSTEP * BPE2 / 2);
#pragma unroll
    for (int q = 0; q < XQ; q++) lds_dma16(rx, b + CT * 1024 + q * 1024, xoff[q] + step * KSTEP * 2);
  };
#pragma unroll
  for (int c = 0; c < R; c++) issue(c, c);

  f32x4_t acc[CT];
#pragma unroll
  for (int t = 0; t < CT; t++) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < SPW; c++) {
    if (c + 1 < SPW) wait_vm<VMS>();
    else wait_vm<0>();
    const uint8_t* b = ring + (c % R) * SLOT;
    u32x4_t wv[CT];
#pragma unroll
    for (int t = 0; t < CT; t++) wv[t] = ld16(b + t * 1024 + lane * 16);
    bf16x8_t xa[MF];
#pragma unroll
    for (int j = 0; j < MF; j++) {
      const int ch = (EPL / 8) * g + j;
      xa[j] = as_bf16x8(ld16(b + CT * 1024 + nl * XRB + 16 * (ch ^ (nl & (CPR - 1)))));
    }
    bf16x8_t bq[CT][4];
#pragma unroll
    for (int t = 0; t < CT; t++) dequant16<WDT>(wv[t], scale_from_raw<WDT>(WDT == W_FP8 ? 0u : svr[c][t]), bq[t]);
    if (c + R < SPW) {
      // the slot's reads have returned before the refill may overwrite it
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(c % R, c + R);
    }
#pragma unroll
    for (int t = 0; t < CT; t++)
#pragma unroll
      for (int j = 0; j < MF; j++) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], bq[t][j], acc[t], 0, 0, 0);
  }

  // acc[t][i] holds C[m = 4g + i][n = nl] of column tile t
  float* red = reinterpret_cast<float*>(smem);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < CT; t++)
#pragma unroll
    for (int i = 0; i < 4; i++) red[((wave * CT + t) * 16 + 4 * g + i) * 16 + nl] = acc[t][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < CT * 256; idx += 64 * NW) {
    const int t = idx >> 8, m = (idx >> 4) & 15, n = idx & 15;
    const int64_t col = n0 + 16 * t + n;
    if (m < M && col < N) {
      float s = 0.0f;
#pragma unroll
      for (int wv = 0; wv < NW; wv++) s += red[((wv * CT + t) * 16 + m) * 16 + n];
      s *= WDT == W_FP8 ? chscale[col] * alpha : alpha;
      y[(int64_t)m * N + col] = (uint16_t)f32_to_bf16_bits(s);
    }
  }
}

// Decode GEMV for 4 < M <= 16, x once per workgroup: every workgroup of the
// ring form reads the whole x (M x K bf16) from L2, as many times as there are
// workgroups, which is more bytes than the weights themselves at M = 16.  Here
// one workgroup of WW waves owns CTW column tiles (16 W rows each) over all of
// K, wave w the K slice [w*KSL, (w+1)*KSL) of SPW steps, so x crosses from L2
// once per workgroup (about once per CU).  Each wave stages the x rows of its
// own slice in a private LDS region by direct-to-LDS loads of whole rows of
// the slice, each row's 16-byte chunks XOR-swizzled by the row so that the 16
// rows of one fragment read sit in distinct banks (x loaded straight into
// registers in the MFMA layout touches two cache lines per row and load: 1 us
// slower at M = 16, no faster at M = 5).  Each lane loads the scales and weight
// chunks of all its steps and tiles into registers up front; the steps then
// convert and multiply in order as the loads land.  The wave partials meet in
// LDS, over the consumed x rows.
template <int WDT, int SPW, int WW, int CTW, int GSH>
__global__ __launch_bounds__(64 * WW) __attribute__((amdgpu_waves_per_eu(WW / 4, WW / 4))) void k_gemv_wide(
    const uint16_t* __restrict__ x, int M, int64_t N, int64_t K, const uint8_t* __restrict__ w,
    const void* __restrict__ sc, const float* __restrict__ chscale, float alpha, uint16_t* __restrict__ y, int cpw) {
  constexpr int EPL = WTraits<WDT>::bits == 4 ? 32 : 16;
  constexpr int KSTEP = 4 * EPL;
  constexpr int KSL = SPW * KSTEP;
  constexpr int MF = EPL / 8;
  constexpr int BPE2 = WTraits<WDT>::bits == 4 ? 1 : 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, g = lane >> 4;
  // the workgroup's cpw columns (a multiple of 8, at most 16 CTW): the rows of
  // its tiles past cpw lie outside the buffer ranges below and read as zeros
  // without a memory access, and their outputs are not stored
  const int64_t n0 = (int64_t)blockIdx.x * cpw;
  const uint32_t rowbytes = (uint32_t)(K * BPE2 / 2);
  const int64_t nrows = N - n0 < cpw ? N - n0 : cpw;
  constexpr int gs = gshift_of<WDT>(GSH);
  const uint32_t spr = (uint32_t)(K >> gs);
  constexpr int SB = scale_bytes<WDT>();
  const auto rw = make_rsrc(w + n0 * rowbytes, nrows * rowbytes);
  const auto rs = make_rsrc(reinterpret_cast<const uint8_t*>(sc) + (WDT == W_FP8 ? 0 : n0 * spr * SB),
                            WDT == W_FP8 ? 0 : nrows * spr * SB);
  const auto rx = make_rsrc(x, (int64_t)M * K * 2);
  const uint32_t kbase = (uint32_t)(wave * KSL);

  // 1) the x rows of the wave's slice (XRB bytes each) at row * XRB of the
  //    wave's region; 16-byte slot p of row r holds the slice's chunk
  //    p ^ (r & 15).  One DMA instruction moves RPD rows.
  constexpr int XRB = KSL * 2, RPD = 1024 / XRB, CPRW = XRB / 16;
  static_assert(XRB <= 1024 && CPRW >= 16, "x slice rows of 256 to 1024 bytes");
  uint8_t* xw = smem + wave * 16 * XRB;
  {
    const int rl = lane / CPRW, p = lane % CPRW;
    for (int i = 0; i * RPD < M; i++) {
      const int r = i * RPD + rl;
      if (r < M) lds_dma16(rx, xw + i * 1024, (uint32_t)(r * (uint32_t)K + kbase) * 2 + 16 * (p ^ (r & 15)));
    }
  }
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // 2) scales and weight chunks of every step into registers, the scales first
  //    (needed by the first conversion); the scheduling barriers keep every
  //    load ahead of the first conversion (the scheduler would otherwise sink
  //    later steps' loads to save registers)
  u32x4_t wr[SPW][CTW];
  uint32_t svr[SPW][CTW];
  const uint32_t wlane = (uint32_t)nl * rowbytes + (kbase + EPL * g) * BPE2 / 2;
  if constexpr (WDT != W_FP8) {
#pragma unroll
    for (int c = 0; c < SPW; c++)
#pragma unroll
      for (int t = 0; t < CTW; t++)
        svr[c][t] = scale_raw_of<WDT>(rs, (uint32_t)(16 * t + nl) * spr + ((kbase + c * KSTEP + EPL * g) >> gs));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < SPW; c++)
#pragma unroll
    for (int t = 0; t < CTW; t++) wr[c][t] = bld16(rw, wlane + 16 * t * rowbytes + c * KSTEP * BPE2 / 2);
  __builtin_amdgcn_sched_barrier(0);
  // this wave's x rows have landed once only the register loads issued after
  // them remain (LDS accesses of one wave execute in order: no barrier)
  wait_vm<SPW * CTW * (WDT == W_FP8 ? 1 : 2)>();
  // MFMA rows >= M read row 0 (their outputs are discarded)
  const int xtr = nl < M ? nl : 0;
  const uint8_t* xrow = xw + xtr * XRB;

  f32x4_t acc[CTW];
#pragma unroll
  for (int t = 0; t < CTW; t++) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto run_steps = [&](auto fast_tag) {
    constexpr bool FASTQ = decltype(fast_tag)::value;
#pragma unroll
    for (int c = 0; c < SPW; c++) {
      bf16x8_t xa[MF];
#pragma unroll
      for (int j = 0; j < MF; j++) {
        const uint32_t q = (c * KSTEP + EPL * g + 8 * j) / 8;
        xa[j] = as_bf16x8(ld16(xrow + 16 * (q ^ (uint32_t)(xtr & 15))));
      }
#pragma unroll
      for (int t = 0; t < CTW; t++) {
        if constexpr (FASTQ && WDT == W_INT4) {
          mma_int4_exact_codes(xa, wr[c][t], bf16_to_f32(svr[c][t]), acc[t]);
        } else {
          bf16x8_t bq[4];
          dequant16<WDT>(wr[c][t], scale_from_raw<WDT>(WDT == W_FP8 ? 0u : svr[c][t]), bq);
#pragma unroll
          for (int j = 0; j < MF; j++) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], bq[j], acc[t], 0, 0, 0);
        }
      }
    }
  };
  // INT4 groups of 128: the exact-code form when every scale of the wave's
  // steps and tiles has a 5-bit significand (decided once the scales, issued
  // before the weights, have landed)
  if constexpr (WDT == W_INT4 && gs == 7) {
    wait_vm<SPW * CTW>();
    bool mine = true;
#pragma unroll
    for (int c = 0; c < SPW; c++)
#pragma unroll
      for (int t = 0; t < CTW; t++) mine &= int4_scale_short(svr[c][t]);
    if (__builtin_amdgcn_ballot_w64(!mine) == 0) run_steps(std::true_type{});
    else run_steps(std::false_type{});
  } else {
    run_steps(std::false_type{});
  }

  // acc[t][i] holds C[m = 4g + i][n = nl] of column tile t; the WW wave
  // partials of every output are added in LDS (over the x rows, once every
  // wave is done with them), one output per thread.  The scheduling barrier
  // keeps the register-only MFMA work ahead of the workgroup barrier (the
  // scheduler may otherwise move it past, and every wave then waits there for
  // the slowest one's loads)
  float* red = reinterpret_cast<float*>(smem);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < CTW; t++)
#pragma unroll
    for (int i = 0; i < 4; i++) red[((wave * CTW + t) * 16 + 4 * g + i) * 16 + nl] = acc[t][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < CTW * 256; idx += 64 * WW) {
    const int t = idx >> 8, m = (idx >> 4) & 15, n = idx & 15;
    const int64_t col = n0 + 16 * t + n;
    if (m < M && col < N && 16 * t + n < cpw) {
      float v = 0.0f;
#pragma unroll
      for (int wv = 0; wv < WW; wv++) v += red[((wv * CTW + t) * 16 + m) * 16 + n];
      v *= WDT == W_FP8 ? chscale[col] * alpha : alpha;
      y[(int64_t)m * N + col] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
}

// Measured on MI355X for K = 4096: 4 waves per 16-column tile with a 2-deep
// ring beat deeper rings (requests all in flight arrive in an order that
// bunches the dequantization work at the end) and 8-wave splits.
constexpr int RING_NW = 4;
// M up to WQ_DECODE_ROWS runs the decode forms, in launches of up to
// WQ_GROUP_ROWS rows (17-32 rows share each converted weight fragment between
// two 16-row MFMA groups)
constexpr int WQ_DECODE_ROWS = 64, WQ_GROUP_ROWS = 32;
// 64 < M <= 256: rows go through the decode launches when this cost model
// says they finish first (at small N and large K the prefill grid leaves most
// CUs idle).  Prefill: ceil(M/256) ceil(N/256) workgroups of one 256x256
// tile, in rounds of one per CU, each tile taking 2 * 256 * 256 * K flops at
// kPrefillTileEff of one CU's bf16 MFMA rate (1024 flops per clock per SIMD,
// 4 SIMDs, at the device's clock).  Decode: one launch per 32 rows, each
// streaming the packed weights at kDecodeRowsHbmFrac of the HBM peak.  The two
// efficiencies are measured on MI355X (a 256x256 tile at K = 4096 takes about
// 90 us: 0.606 of the CU rate; a 32-row launch moves 29.4 MB in about 20 us:
// 0.1875 of 8 TB/s); the CU count and clock come from the device.
constexpr double kPrefillTileEff = 0.606, kDecodeRowsHbmFrac = 0.1875, kHbmPeakBytesPerS = 8.0e12;
struct DeviceRates { int ncu; double clk_hz; };
hipError_t device_rates(DeviceRates* out) {
  static DeviceRates cached[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cached[dev].ncu > 0) {
    *out = cached[dev];
    return hipSuccess;
  }
  int ncu = 0, khz = 0;
  if ((e = cu_count(&ncu)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev)) != hipSuccess) return e;
  DeviceRates r{ncu, khz > 0 ? khz * 1e3 : 2.4e9};
  if (dev >= 0 && dev < 64) cached[dev] = r;
  *out = r;
  return hipSuccess;
}
inline bool decode_rows_pay(int64_t M, int64_t N, int64_t K, int bits, const DeviceRates& r) {
  const int64_t wgs = ((M + 255) / 256) * ((N + 255) / 256);
  const double tile_s = 2.0 * 256 * 256 * (double)K / (4.0 * 1024.0 * r.clk_hz * kPrefillTileEff);
  const double t_pre = (double)((wgs + r.ncu - 1) / r.ncu) * tile_s;
  const double t_dec = (double)((M + 31) / 32) * (double)N * (double)K * bits / 8 / (kDecodeRowsHbmFrac * kHbmPeakBytesPerS);
  return t_dec < t_pre;
}
constexpr int RING_DEPTH = 2;
// 4 < M <= 16: two 16-column tiles per workgroup share every x chunk, which
// halves the x traffic from L2 (each workgroup reads the whole x slice).
constexpr int RING16_CT = 2, RING16_NW = 4;
template <int WDT, int SPW, int GSH>
wq_status ring16_go(int64_t M, const uint16_t* x, int64_t N, int64_t K, const uint8_t* w, const void* sc,
                    const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  constexpr int R = SPW < 2 ? SPW : 2;
  if constexpr (R < 2) {
    return WQ_EUNSUPPORTED;
  } else {
    constexpr int CT = RING16_CT;
    constexpr int XSLOT = 16 * 4 * (WTraits<WDT>::bits == 4 ? 32 : 16) * 2;
    constexpr int NW = RING16_NW;
    const size_t lds = (size_t)NW * R * (CT * 1024 + XSLOT);
    const unsigned grid = (unsigned)((N + 16 * CT - 1) / (16 * CT));
    if (allow_lds<k_gemv_ring16<WDT, SPW, R, NW, CT, GSH>>(lds) != hipSuccess) return WQ_EHIP;
    k_gemv_ring16<WDT, SPW, R, NW, CT, GSH><<<grid, 64 * NW, lds, s>>>(x, (int)M, N, K, w, sc, ch, alpha, y);
    return WQ_OK;
  }
}

// x-once form: 16 waves x 4 column tiles per workgroup, K = 2048 or 4096
// (1 or 2 steps per wave for 4-bit weights, 2 or 4 for E4M3)
constexpr int WIDE_WW = 16, WIDE_CTW = 4;
template <int WDT, int SPW, int GSH>
wq_status wide_go(int64_t M, const uint16_t* x, int64_t N, int64_t K, const uint8_t* w, const void* sc,
                  const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  // x: 16 rows of the wave's slice per wave (K * 2 * 16 bytes in all); the
  // partials reuse it
  const size_t red = (size_t)WIDE_WW * WIDE_CTW * 1024, xb = (size_t)16 * K * 2;
  const size_t lds = xb > red ? xb : red;
  // columns per workgroup: 16 CTW, or fewer (a multiple of 8) when that
  // leaves CUs idle, so that the workgroups cover the CUs once (N = 14336:
  // 256 workgroups of 56 columns instead of 224 of 64)
  int ncu = 0;
  if (cu_count(&ncu) != hipSuccess) return WQ_EHIP;
  int64_t cpw = 16 * WIDE_CTW;
  if ((N + cpw - 1) / cpw < ncu) {
    const int64_t c = ((N + ncu - 1) / ncu + 7) / 8 * 8;
    cpw = c < 8 ? 8 : (c > cpw ? cpw : c);
  }
  const unsigned grid = (unsigned)((N + cpw - 1) / cpw);
  if (allow_lds<k_gemv_wide<WDT, SPW, WIDE_WW, WIDE_CTW, GSH>>(lds) != hipSuccess) return WQ_EHIP;
  k_gemv_wide<WDT, SPW, WIDE_WW, WIDE_CTW, GSH><<<grid, 64 * WIDE_WW, lds, s>>>(x, (int)M, N, K, w, sc, ch, alpha, y,
                                                                              (int)cpw);
  return WQ_OK;
}

template <int WDT, int SPW, int R, int GSH, bool XS>
wq_status ring_launch(int64_t M, const uint16_t* x, int64_t N, int64_t K, const uint8_t* w, const void* sc,
                      const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  const int full = ring_wave_bytes<WDT, GSH>(SPW, R, false, XS, (int)M);
  const int half = SPW >= 2 ? ring_wave_bytes<WDT, GSH>(SPW / 2, ring_half_depth(SPW, R, XS), true, XS, (int)M) : 0;
  // at least the split-K reduction's 16 x 16 fp32 partials per wave
  const int wave_bytes = full > half ? full : half;
  const size_t lds = (size_t)RING_NW * (wave_bytes > 1024 ? wave_bytes : 1024);
  if (allow_lds<k_gemv_ring<WDT, SPW, R, RING_NW, GSH, XS>>(lds) != hipSuccess) return WQ_EHIP;
  // all tiles are resident at once and dispatched round by round over the
  // CUs; a last round that covers at most half of the CUs becomes twice as
  // many 8-column tiles, one per CU
  const int64_t tiles = (N + 15) / 16;
  int ncu = 0;
  if (cu_count(&ncu) != hipSuccess) return WQ_EHIP;
  const int64_t last = tiles % ncu;
  const int64_t nfull = SPW >= 2 && last > 0 && 2 * last <= ncu ? tiles - last : tiles;
  const unsigned grid = (unsigned)(nfull + 2 * (tiles - nfull));
  k_gemv_ring<WDT, SPW, R, RING_NW, GSH, XS><<<grid, 64 * RING_NW, lds, s>>>(x, (int)M, N, K, w, sc, ch, alpha, y,
                                                                           (int)nfull);
  return WQ_OK;
}

// Loads run RING_DEPTH steps ahead for up to three tokens; with four tokens
// the steps take longer and a deeper ring keeps more bytes in flight (measured
// at M = 4: one more step for 4-bit weights, two more for 8-bit; at M = 3 the
// shallow ring is faster, 10.7 against 11.6 us for INT4).
template <int WDT, int SPW, int GSH>
wq_status ring_go(int64_t M, const uint16_t* x, int64_t N, int64_t K, const uint8_t* w, const void* sc,
                  const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  constexpr int R1 = SPW < RING_DEPTH ? SPW : RING_DEPTH;
  constexpr int RM0 = RING_DEPTH + (WTraits<WDT>::bits == 8 ? 2 : 1);
  constexpr int RM = SPW < RM0 ? SPW : RM0;
  // four tokens of 4-bit weights: x through the ring slots (measured 8 % faster
  // there, 4 % slower for E4M3)
  constexpr bool XS4 = WTraits<WDT>::bits == 4;
  if (M <= 3) return ring_launch<WDT, SPW, R1, GSH, false>(M, x, N, K, w, sc, ch, alpha, y, s);
  return ring_launch<WDT, SPW, RM, GSH, XS4>(M, x, N, K, w, sc, ch, alpha, y, s);
}

// The ring forms, when K splits into 4 wave slices of 1, 2, 4, 8 or 16 steps;
// false when the shape needs the general GEMV.
template <int WDT, int GSH>
bool ring_path(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w, const void* sc,
               const float* ch, float alpha, uint16_t* y, hipStream_t s, wq_status& st) {
  constexpr int KSTEP = WTraits<WDT>::bits == 4 ? 128 : 64;
  if (K % (KSTEP * RING_NW) || 16 * K * 2 > 0x7FFFFFF0LL) return false;
  const int64_t spw = K / (KSTEP * RING_NW);
  if (M <= 4) {
    // (8 or 16 waves per tile when the tiles are few, each with a shorter K
    // slice, measured no faster: N = 4096, K = 4096: 5.4 against 5.2-5.4 us;
    // N = 8192: 7.6 against 6.6 us)
    switch (spw) {
      case 1: st = ring_go<WDT, 1, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;
      case 2: st = ring_go<WDT, 2, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;
      case 4: st = ring_go<WDT, 4, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;
      case 8: st = ring_go<WDT, 8, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;
      case 16: st = ring_go<WDT, 16, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;
      case 28: st = ring_go<WDT, 28, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;   // K = 14336, 4-bit
      default: return false;
    }
  }
  // when the 16-column tiles alone do not fill the CUs, the general form
  // (one tile and up to 16 waves per workgroup) is faster for 4 < M <= 16
  // (measured N = 1024-4096: 7.9-8.9 us against 11.3-12.1 us)
  if (M > 16) return false;
  int ncu = 0;
  if (cu_count(&ncu) != hipSuccess) {
    st = WQ_EHIP;
    return true;
  }
  if ((N + 15) / 16 <= ncu) return false;
  constexpr int SW = WTraits<WDT>::bits == 4 ? 1 : 2;          // steps per wave at K = 2048
  if (K == 2048) { st = wide_go<WDT, SW, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true; }
  if (K == 4096) { st = wide_go<WDT, 2 * SW, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true; }
  if (K % (KSTEP * RING16_NW)) return false;
  switch (K / (KSTEP * RING16_NW)) {
    case 2: st = ring16_go<WDT, 2, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;
    case 4: st = ring16_go<WDT, 4, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;
    case 8: st = ring16_go<WDT, 8, GSH>(M, x, N, K, w, sc, ch, alpha, y, s); return true;
    // (longer K: two tiles per workgroup with x through LDS measured faster,
    // N = 8192, K = 8192: 16.0 -> 14.7 us at M = 5 and 8)
    default: return false;
  }
}

template <int WDT>
wq_status launch_gemv(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w, const void* sc, int group,
                      const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  constexpr int KSTEP = WTraits<WDT>::bits == 4 ? 128 : 64;
  wq_status st = WQ_OK;
  bool ring;
  if constexpr (WDT == W_INT4 || WDT == W_UINT4) {
    ring = group == 32   ? ring_path<WDT, 5>(x, M, N, K, w, sc, ch, alpha, y, s, st)
           : group == 64 ? ring_path<WDT, 6>(x, M, N, K, w, sc, ch, alpha, y, s, st)
                         : ring_path<WDT, 7>(x, M, N, K, w, sc, ch, alpha, y, s, st);
  } else {
    ring = ring_path<WDT, 0>(x, M, N, K, w, sc, ch, alpha, y, s, st);
  }
  if (ring) return st != WQ_OK ? st : wq_launch_status();
  constexpr int MAXSTEP = WTraits<WDT>::bits == 4 ? 4 : 8;
  // the per-workgroup buffer resources address 16*TN rows (< 2^31 bytes)
  if (32 * K * (WTraits<WDT>::bits / 4) / 2 > 0x7FFFFFF0LL || M * K * 2 > 0x7FFFFFF0LL) return WQ_EINVAL;
  if (K % KSTEP) {
    // K = 128*j with j odd only matters for 8-bit weights, whose step is 64: always divisible
    return WQ_EINVAL;
  }
  // up to 16 waves per workgroup when the column tiles alone do not fill the CUs
  int ncu = 0;
  if (cu_count(&ncu) != hipSuccess) return WQ_EHIP;
  const int64_t tiles = (N + 15) / 16;
  hipError_t e;
  if (M <= 4) {
    e = gemv_nstep<WDT>(gemv_split(K / KSTEP, MAXSTEP, tiles <= ncu ? 16 : 8), x, M, N, K, w, sc, group, ch, alpha,
                        y, s);
  } else {
    // x through LDS, one chunk row's 16-byte x pieces in groups of 16 (one
    // step for 4-bit weights, two for 8-bit: their step count is even since
    // K % 128 == 0; one step measured faster than two for 4-bit, N = 1792-8192,
    // K = 4096-14336, M = 5-16).  Two 16-column tiles per workgroup when the
    // tiles outnumber the CUs, so that x is fetched once per 32 columns
    // (N = 8192, K = 14336, M = 16: 29.6 -> 25.5 us).
    constexpr int XS = WTraits<WDT>::bits == 4 ? 1 : 2;
    const bool t2 = tiles > ncu;
    // (two tiles and 32 rows need more than 128 registers per lane: at most 8
    // waves per workgroup)
    const bool s16 = (t2 ? (tiles + 1) / 2 : tiles) <= ncu && !(t2 && M > 16);
    const GemvSplit sx = gemv_split(K / KSTEP, XS, s16 ? 16 : 8);
    if (sx.nstep != XS) return WQ_EINVAL;
    if (M > 16)
      e = t2 ? x16_go<WDT, XS, 2, 2>(sx, x, M, N, K, w, sc, group, ch, alpha, y, s)
             : x16_go<WDT, XS, 1, 2>(sx, x, M, N, K, w, sc, group, ch, alpha, y, s);
    else
      e = t2 ? x16_go<WDT, XS, 2, 1>(sx, x, M, N, K, w, sc, group, ch, alpha, y, s)
             : x16_go<WDT, XS, 1, 1>(sx, x, M, N, K, w, sc, group, ch, alpha, y, s);
  }
  return e != hipSuccess ? WQ_EHIP : wq_launch_status();
}

template <int WDT>
wq_status launch_gemm(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w, const void* sc, int group,
                      const float* ch, float alpha, uint16_t* y, hipStream_t s) {
  using C8 = Gemm8<WDT>;
  // 32-bit buffer offsets: one 256-row x tile, one 256-row W tile, one 256-row y tile
  if ((int64_t)C8::BM * K * 2 > 0x7FFFFFF0LL || (int64_t)C8::BM * N * 2 > 0x7FFFFFF0LL) return WQ_EINVAL;
  if (allow_lds<k_gemm8<WDT>>(C8::LDS) != hipSuccess) return WQ_EHIP;
  const int tm = (int)((M + C8::BM - 1) / C8::BM), tn = (int)((N + C8::BN - 1) / C8::BN);
  const int gshift = group == 32 ? 5 : group == 64 ? 6 : 7;
  k_gemm8<WDT><<<(unsigned)(tm * tn), 64 * C8::NW, C8::LDS, s>>>(x, M, N, K, w, sc, gshift, ch, alpha, y, tm, tn);
  return wq_launch_status();
}

}  // namespace

extern "C" {

size_t wq_gemm_workspace_size(int64_t, int64_t, int64_t, int, int32_t) { return 0; }

wq_status wq_gemm(const void* x_bf16, int64_t M, int64_t N, int64_t K, const void* wqp, int w_dtype,
                  const void* w_scales, int s_dtype, int32_t group, float alpha, void* y_bf16, void* workspace,
                  size_t ws_bytes, void* stream) {
  (void)workspace;
  (void)ws_bytes;
  if (!x_bf16 || !wqp || !w_scales || !y_bf16) return WQ_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || K % 128) return WQ_EINVAL;
  if (!(alpha == alpha) || alpha > 3.4028234e38f || alpha < -3.4028234e38f) return WQ_EINVAL;
  if (!wq_numel_ok(M, K) || !wq_numel_ok(N, K) || !wq_numel_ok(M, N) || M > 0x7FFFFFFF) return WQ_EINVAL;
  if (!wq_aligned(x_bf16) || !wq_aligned(wqp) || !wq_aligned(y_bf16)) return WQ_EALIGN;
  int wdt;
  if (w_dtype == WQ_INT4X8 && s_dtype == WQ_BF16 && (group == 32 || group == 64 || group == 128)) wdt = W_INT4;
  else if (w_dtype == WQ_E2M1X2 && s_dtype == WQ_E8M0 && group == 32) wdt = W_FP4;
  else if (w_dtype == WQ_E2M1X2 && s_dtype == WQ_E4M3 && group == 16) wdt = W_NV4;
  else if (w_dtype == WQ_UINT4X8 && s_dtype == WQ_BF16Z && (group == 32 || group == 64 || group == 128)) wdt = W_UINT4;
  else if (w_dtype == WQ_E4M3 && s_dtype == WQ_F32 && group == K) wdt = W_FP8;
  else return WQ_EUNSUPPORTED;
  if (M > 16 && (int64_t)((M + 255) / 256) * ((N + 255) / 256) > 0x7FFFFFFF) return WQ_EINVAL;   // prefill tiles
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* x = (const uint16_t*)x_bf16;
  const uint8_t* w = (const uint8_t*)wqp;
  uint16_t* y = (uint16_t*)y_bf16;
  const float* ch = wdt == W_FP8 ? (const float*)w_scales : nullptr;
  // M <= 16: the decode forms.  16 < M <= 64: the GEMM's 256-row tiles leave
  // most CUs idle (N / 256 workgroups: 90 us at N = 14336, K = 4096 for any
  // M up to 512), so the rows go through the decode forms in launches of up
  // to 32 rows, each streaming the weights once (about 20 us per 32 rows
  // there).
  bool rows = M <= WQ_DECODE_ROWS;
  if (!rows && M <= 256) {
    DeviceRates dr{};
    if (device_rates(&dr) != hipSuccess) return WQ_EHIP;
    rows = decode_rows_pay(M, N, K, wdt == W_FP8 ? 8 : 4, dr);
  }
  if (rows) {
    for (int64_t m0 = 0; m0 < M; m0 += WQ_GROUP_ROWS) {
      const int64_t mg = M - m0 < WQ_GROUP_ROWS ? M - m0 : WQ_GROUP_ROWS;
      const uint16_t* xg = x + m0 * K;
      uint16_t* yg = y + m0 * N;
      wq_status st;
      switch (wdt) {
        case W_INT4: st = launch_gemv<W_INT4>(xg, mg, N, K, w, w_scales, group, ch, alpha, yg, s); break;
        case W_FP4: st = launch_gemv<W_FP4>(xg, mg, N, K, w, w_scales, group, ch, alpha, yg, s); break;
        case W_NV4: st = launch_gemv<W_NV4>(xg, mg, N, K, w, w_scales, group, ch, alpha, yg, s); break;
        case W_UINT4: st = launch_gemv<W_UINT4>(xg, mg, N, K, w, w_scales, group, ch, alpha, yg, s); break;
        default: st = launch_gemv<W_FP8>(xg, mg, N, K, w, w_scales, group, ch, alpha, yg, s); break;
      }
      if (st != WQ_OK) return st;
    }
    return WQ_OK;
  }
  switch (wdt) {
    case W_INT4: return launch_gemm<W_INT4>(x, M, N, K, w, w_scales, group, ch, alpha, y, s);
    case W_FP4: return launch_gemm<W_FP4>(x, M, N, K, w, w_scales, group, ch, alpha, y, s);
    case W_NV4: return launch_gemm<W_NV4>(x, M, N, K, w, w_scales, group, ch, alpha, y, s);
    case W_UINT4: return launch_gemm<W_UINT4>(x, M, N, K, w, w_scales, group, ch, alpha, y, s);
    default: return launch_gemm<W_FP8>(x, M, N, K, w, w_scales, group, ch, alpha, y, s);
  }
}

}  // extern "C"

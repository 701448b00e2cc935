// Weight-only quantized matmul y[M,N] = x[M,K] . dequant(W[N,K])^T for gfx950.
//
// Decode (M <= 16): split-K GEMV.  A workgroup owns 16*TN output columns and
// S waves; wave w streams the K-slice [w*K/S, (w+1)*K/S) of those rows with
// 16-byte loads issued up front, converts the packed weights to bf16 in
// registers and feeds v_mfma_f32_16x16x32_bf16 (x rows beyond M are zero).
// The S partial 16x16 tiles are reduced through LDS and rounded to bf16 once.
//
// Prefill (M > 16): 256x256 output tile per workgroup, 4 waves of 128x128,
// K step 64 with double-buffered LDS tiles (x in bf16, W still packed); each
// wave dequantizes its W fragments from LDS in registers right before
// v_mfma_f32_32x32x16_bf16.
#include <hip/hip_runtime.h>

#include "wq.h"
#include "wq_device.h"
#include "wq_host.h"

using namespace wq;

namespace {

enum { W_INT4 = 0, W_FP4 = 1, W_FP8 = 2 };

template <int WDT> struct WTraits;
template <> struct WTraits<W_INT4> { static constexpr int bits = 4; };
template <> struct WTraits<W_FP4> { static constexpr int bits = 4; };
template <> struct WTraits<W_FP8> { static constexpr int bits = 8; };

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{a, b, c, d});
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Per-lane scale operand for a 32-element K slice starting at k.
template <int WDT>
__device__ __forceinline__ float load_scale(const void* sc, int64_t row, int64_t K, int group, int64_t k) {
  if constexpr (WDT == W_INT4) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(sc)[row * (K / group) + k / group]);
  } else if constexpr (WDT == W_FP4) {
    return e8m0_as_scale(reinterpret_cast<const uint8_t*>(sc)[row * (K / 32) + k / 32]);
  } else {
    return 1.0f;
  }
}

// Convert one packed 16-byte weight chunk to bf16 MFMA operands.
// 4-bit: 32 elements -> 4 operands of 8; 8-bit: 16 elements -> 2 operands.
template <int WDT>
__device__ __forceinline__ void dequant16(u32x4_t w, float s, bf16x8_t out[4]) {
  if constexpr (WDT == W_INT4) {
    if (int4_scale_fast(s)) {
      const Int4Consts c = int4_consts(s);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        uint32_t o[4];
        dq_int4_word(w[j], c, o);
        out[j] = as_bf16x8(o[0], o[1], o[2], o[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        uint32_t o[4];
        dq_int4_word_direct(w[j], s, o);
        out[j] = as_bf16x8(o[0], o[1], o[2], o[3]);
      }
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

// ---------------------------------------------------------------------------
// Decode GEMV
// ---------------------------------------------------------------------------
template <int WDT, int TN, int CH>
__global__ __launch_bounds__(512) void k_gemv(const uint16_t* __restrict__ x, int M, int64_t N, int64_t K,
                                             const uint8_t* __restrict__ w, const void* __restrict__ sc, int group,
                                             const float* __restrict__ chscale, uint16_t* __restrict__ y, int kw) {
  constexpr int EPL = WTraits<WDT>::bits == 4 ? 32 : 16;   // elements per lane per step
  constexpr int KSTEP = 4 * EPL;                            // K covered by a wave per step
  constexpr int MF = EPL / 8;                               // MFMAs per step per tile
  constexpr int BPE2 = WTraits<WDT>::bits == 4 ? 1 : 2;     // bytes per 2 elements
  extern __shared__ float red[];                            // [S][TN][16][16]

  const int S = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * TN;
  const int64_t kbeg = (int64_t)wave * kw, kend = kbeg + kw;
  const int64_t rowbytes = K * BPE2 / 2;

  int64_t nrow[TN];
#pragma unroll
  for (int t = 0; t < TN; t++) {
    const int64_t n = n0 + 16 * t + nl;
    nrow[t] = n < N ? n : N - 1;                 // clamped: always a valid row
  }
  const bool xrow = nl < M;                      // this lane carries a real x row
  const uint16_t* xr = x + (int64_t)(xrow ? nl : 0) * K;

  f32x4_t acc[TN];
#pragma unroll
  for (int t = 0; t < TN; t++) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kbeg; k0 < kend; k0 += (int64_t)CH * KSTEP) {
    u32x4_t wr[CH][TN];
    float sv[CH][TN];
#pragma unroll
    for (int c = 0; c < CH; c++) {
      const int64_t kk = k0 + (int64_t)c * KSTEP + (int64_t)EPL * g;
      if (k0 + (int64_t)c * KSTEP < kend) {
#pragma unroll
        for (int t = 0; t < TN; t++) {
          wr[c][t] = ld16(w + nrow[t] * rowbytes + kk * BPE2 / 2);
          sv[c][t] = load_scale<WDT>(sc, nrow[t], K, group, kk);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; c++) {
      if (k0 + (int64_t)c * KSTEP >= kend) break;
      const int64_t kk = k0 + (int64_t)c * KSTEP + (int64_t)EPL * g;
      bf16x8_t xa[MF];
#pragma unroll
      for (int j = 0; j < MF; j++) {
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (xrow) v = ld16(xr + kk + 8 * j);
        xa[j] = as_bf16x8(v);
      }
#pragma unroll
      for (int t = 0; t < TN; t++) {
        bf16x8_t b[4];
        dequant16<WDT>(wr[c][t], sv[c][t], b);
#pragma unroll
        for (int j = 0; j < MF; j++) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], b[j], acc[t], 0, 0, 0);
      }
    }
  }

  // acc[t][i] holds C[m = 4g + i][n = nl] of tile t.
#pragma unroll
  for (int t = 0; t < TN; t++)
#pragma unroll
    for (int i = 0; i < 4; i++) red[((wave * TN + t) * 16 + 4 * g + i) * 16 + nl] = acc[t][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < TN * 256; idx += blockDim.x) {
    const int t = idx >> 8, m = (idx >> 4) & 15, n = idx & 15;
    const int64_t col = n0 + 16 * t + n;
    if (m >= M || col >= N) continue;
    float s = 0.0f;
    for (int wv = 0; wv < S; wv++) s += red[((wv * TN + t) * 16 + m) * 16 + n];
    if constexpr (WDT == W_FP8) s *= chscale[col];
    y[(int64_t)m * N + col] = (uint16_t)f32_to_bf16_bits(s);
  }
}

// ---------------------------------------------------------------------------
// Prefill GEMM
// ---------------------------------------------------------------------------
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int A_STRIDE = BK * 2 + 16;                  // bytes per x row in LDS (padded)

template <int WDT>
struct GemmCfg {
  static constexpr int wbytes = BK * WTraits<WDT>::bits / 8;   // packed bytes per W row per K step
  static constexpr int B_STRIDE = wbytes + 16;                  // padded
  static constexpr int A_TILE = BM * A_STRIDE;
  static constexpr int B_TILE = BN * B_STRIDE;
  static constexpr int STAGE = A_TILE + B_TILE;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int B_CHUNKS = BN * wbytes / 16 / 256;       // 16-byte chunks per thread
};

template <int WDT>
__global__ __launch_bounds__(256) void k_gemm(const uint16_t* __restrict__ x, int64_t M, int64_t N, int64_t K,
                                             const uint8_t* __restrict__ w, const void* __restrict__ sc, int group,
                                             const float* __restrict__ chscale, uint16_t* __restrict__ y,
                                             int tiles_m, int tiles_n) {
  using C = GemmCfg<WDT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;

  // XCD-aware order: consecutive workgroup ids land on different XCDs, so give
  // each XCD a contiguous range of tiles (m-major, which shares B panels).
  const int nwg = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if (nwg % 8 == 0) pid = (pid % 8) * (nwg / 8) + pid / 8;
  const int tn = pid % tiles_n, tm = pid / tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t rowbytes = K * WTraits<WDT>::bits / 8;

  // global -> LDS copy assignments
  // x: 256 rows x 128 B: thread covers rows (tid/8) + 32*i, 16-byte chunk tid%8
  const int a_row = tid >> 3, a_chk = tid & 7;
  const uint16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    int64_t r = m0 + a_row + 32 * i;
    r = r < M ? r : M - 1;
    a_src[i] = x + r * K + a_chk * 8;
  }
  // W: BN rows x wbytes: chunks per row = wbytes/16
  constexpr int CPR = C::wbytes / 16;
  const uint8_t* b_src[C::B_CHUNKS];
  int b_dst[C::B_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; i++) {
    const int q = tid + 256 * i;
    const int r = q / CPR, ch = q % CPR;
    int64_t n = n0 + r;
    n = n < N ? n : N - 1;
    b_src[i] = w + n * rowbytes + ch * 16;
    b_dst[i] = r * C::B_STRIDE + ch * 16;
  }
  // scale rows of this lane's four n-subtiles
  int64_t srow[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    int64_t n = n0 + wn * 128 + 32 * j + l32;
    srow[j] = n < N ? n : N - 1;
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  u32x4_t ra[8], rb[C::B_CHUNKS];
  float rs[4], cs[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 8; i++) ra[i] = ld16(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; i++) rb[i] = ld16(b_src[i] + k0 * WTraits<WDT>::bits / 8);
#pragma unroll
    for (int j = 0; j < 4; j++) rs[j] = load_scale<WDT>(sc, srow[j], K, group, k0 + 32 * h);
  };
  auto lstore = [&](int stage) {
    uint8_t* A = lds + stage * C::STAGE;
    uint8_t* B = A + C::A_TILE;
#pragma unroll
    for (int i = 0; i < 8; i++) *reinterpret_cast<u32x4_t*>(A + (a_row + 32 * i) * A_STRIDE + a_chk * 16) = ra[i];
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; i++) *reinterpret_cast<u32x4_t*>(B + b_dst[i]) = rb[i];
  };

  const int nk = (int)(K / BK);
  gload(0);
  lstore(0);
#pragma unroll
  for (int j = 0; j < 4; j++) cs[j] = rs[j];
  __syncthreads();

  for (int kt = 0; kt < nk; kt++) {
    const int stage = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * BK);
    const uint8_t* A = lds + stage * C::STAGE;
    const uint8_t* B = A + C::A_TILE;
    // packed W fragments of this lane for the whole K step
    bf16x8_t bq[4][4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint8_t* bp = B + (wn * 128 + 32 * j + l32) * C::B_STRIDE;
      if constexpr (WTraits<WDT>::bits == 4) {
        const u32x4_t pw = *reinterpret_cast<const u32x4_t*>(bp + 16 * h);
        dequant16<WDT>(pw, cs[j], bq[j]);
      } else {
        const u32x4_t p0 = *reinterpret_cast<const u32x4_t*>(bp + 32 * h);
        const u32x4_t p1 = *reinterpret_cast<const u32x4_t*>(bp + 32 * h + 16);
        dequant16<WDT>(p0, 1.0f, bq[j]);
        dequant16<WDT>(p1, 1.0f, bq[j] + 2);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; s++) {
      bf16x8_t af[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(A + (wm * 128 + 32 * i + l32) * A_STRIDE + (32 * h + 8 * s) * 2));
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bq[j][s], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      __syncthreads();           // everyone is done reading the other stage
      lstore(stage ^ 1);
#pragma unroll
      for (int j = 0; j < 4; j++) cs[j] = rs[j];
      __syncthreads();
    }
  }

  // epilogue: C element r of a 32x32 tile sits at row 8*(r/4) + 4*h + r%4, col l32
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int64_t col = n0 + wn * 128 + 32 * j + l32;
    if (col >= N) continue;
    float cscale = 1.0f;
    if constexpr (WDT == W_FP8) cscale = chscale[col];
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < M) y[row * N + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][r] * cscale);
      }
    }
  }
}

template <int WDT>
wq_status launch_gemv(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w, const void* sc, int group,
                      const float* ch, uint16_t* y, hipStream_t s) {
  constexpr int KSTEP = WTraits<WDT>::bits == 4 ? 128 : 64;
  constexpr int CH = WTraits<WDT>::bits == 4 ? 4 : 8;
  int S = 8;
  while (S > 1 && (K % ((int64_t)S * KSTEP) != 0)) S >>= 1;
  if (K % ((int64_t)S * KSTEP) != 0) return WQ_EINVAL;
  const int kw = (int)(K / S);
  if (M <= 4) {
    constexpr int TN = 1;
    const unsigned grid = (unsigned)((N + 16 * TN - 1) / (16 * TN));
    k_gemv<WDT, TN, CH><<<grid, 64 * S, S * TN * 1024, s>>>(x, (int)M, N, K, w, sc, group, ch, y, kw);
  } else {
    constexpr int TN = 2;
    const unsigned grid = (unsigned)((N + 16 * TN - 1) / (16 * TN));
    k_gemv<WDT, TN, CH><<<grid, 64 * S, S * TN * 1024, s>>>(x, (int)M, N, K, w, sc, group, ch, y, kw);
  }
  return wq_launch_status();
}

template <int WDT>
wq_status launch_gemm(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* w, const void* sc, int group,
                      const float* ch, uint16_t* y, hipStream_t s) {
  using C = GemmCfg<WDT>;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_gemm<WDT>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS) !=
        hipSuccess)
      return WQ_EHIP;
    attr_set = true;
  }
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  k_gemm<WDT><<<(unsigned)(tm * tn), 256, C::LDS, s>>>(x, M, N, K, w, sc, group, ch, y, tm, tn);
  return wq_launch_status();
}

}  // namespace

extern "C" {

size_t wq_gemm_workspace_size(int64_t, int64_t, int64_t, int, int32_t) { return 0; }

wq_status wq_gemm(const void* x_bf16, int64_t M, int64_t N, int64_t K, const void* wqp, int w_dtype,
                  const void* w_scales, int s_dtype, int32_t group, void* y_bf16, void* workspace, size_t ws_bytes,
                  void* stream) {
  (void)workspace;
  (void)ws_bytes;
  if (!x_bf16 || !wqp || !w_scales || !y_bf16) return WQ_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || K % 128) return WQ_EINVAL;
  if (!wq_numel_ok(M, K) || !wq_numel_ok(N, K) || !wq_numel_ok(M, N) || M > 0x7FFFFFFF) return WQ_EINVAL;
  if (!wq_aligned(x_bf16) || !wq_aligned(wqp) || !wq_aligned(y_bf16)) return WQ_EALIGN;
  int wdt;
  if (w_dtype == WQ_INT4X8 && s_dtype == WQ_BF16 && (group == 32 || group == 64 || group == 128)) wdt = W_INT4;
  else if (w_dtype == WQ_E2M1X2 && s_dtype == WQ_E8M0 && group == 32) wdt = W_FP4;
  else if (w_dtype == WQ_E4M3 && s_dtype == WQ_F32 && group == K) wdt = W_FP8;
  else return WQ_EUNSUPPORTED;
  if (M > 16 && (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN) > 0x7FFFFFFF) return WQ_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* x = (const uint16_t*)x_bf16;
  const uint8_t* w = (const uint8_t*)wqp;
  uint16_t* y = (uint16_t*)y_bf16;
  const float* ch = wdt == W_FP8 ? (const float*)w_scales : nullptr;
  if (M <= 16) {
    switch (wdt) {
      case W_INT4: return launch_gemv<W_INT4>(x, M, N, K, w, w_scales, group, ch, y, s);
      case W_FP4: return launch_gemv<W_FP4>(x, M, N, K, w, w_scales, group, ch, y, s);
      default: return launch_gemv<W_FP8>(x, M, N, K, w, w_scales, group, ch, y, s);
    }
  }
  switch (wdt) {
    case W_INT4: return launch_gemm<W_INT4>(x, M, N, K, w, w_scales, group, ch, y, s);
    case W_FP4: return launch_gemm<W_FP4>(x, M, N, K, w, w_scales, group, ch, y, s);
    default: return launch_gemm<W_FP8>(x, M, N, K, w, w_scales, group, ch, y, s);
  }
}

}  // extern "C"

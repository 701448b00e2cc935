// W8A8 FP8 for gfx950: the per-tensor static E4M3 activation quantizer, the
// 128 x 128 block E4M3 weight quantizer, and the GEMM
// y[M,N] = sum over 128-wide K blocks of (a_s * b_s) * (a . b) with fp32
// accumulation on the fp8 matrix cores and one bf16 rounding at the store.
#include <hip/hip_runtime.h>

#include "wq.h"
#include "wq_device.h"
#include "wq_host.h"

using namespace wq;

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
inline unsigned grid_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

// RN(x / s) for s in [2^-90, 2^90] given y = RN(1 / s); quotients beyond
// 512 saturate anyway and keep the first estimate (the correction step would
// turn an infinite estimate into NaN).
__device__ __forceinline__ float quot_sat(float x, float s, float y) {
  const float q0 = x * y;
  return __builtin_fabsf(q0) > 512.0f ? q0 : div_rn_markstein(x, s, y);
}

// ---------------------------------------------------------------------------
// Per-tensor static quantizer: 16 elements per thread, one fp32 scale read
// from device memory.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_e4m3_static(const void* __restrict__ x, int64_t nchunks,
                                                         const float* __restrict__ scale, uint8_t* __restrict__ codes) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= nchunks) return;
  const float s = scale[0];
  float v[16];
  load8<BF16>(x, t * 16, v);
  load8<BF16>(x, t * 16 + 8, v + 8);
  float q[16];
  if (s >= 0x1p-90f && s <= 0x1p90f) {
    const float y = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 16; i++) q[i] = clamp448(quot_sat(v[i], s, y));
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) q[i] = clamp448(v[i] / s);
  }
  u32x4_t out;
#pragma unroll
  for (int d = 0; d < 4; d++) {
    const uint32_t r = e4m3_pack2<false>(q[4 * d], q[4 * d + 1], 0u);
    out[d] = e4m3_pack2<true>(q[4 * d + 2], q[4 * d + 3], r);
  }
  *reinterpret_cast<u32x4_t*>(codes + t * 16) = out;
}

// ---------------------------------------------------------------------------
// 128 x 128 block quantizer: one workgroup per block; thread t holds 64
// elements of row t / 2 (columns 64 (t % 2) .. +64).  s = RN(amax / 448),
// 1 if zero; codes e4m3(RN(w / s)).  Rows past N read as zero and are not
// stored.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_e4m3_block2d(const void* __restrict__ w, int64_t N, int64_t K,
                                                          uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[kThreads / 64];
  const int t = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.y * 128 + (t >> 1);
  const int64_t col = (int64_t)blockIdx.x * 128 + 64 * (t & 1);
  const bool live = row < N;
  float v[64];
  if (live) {
#pragma unroll
    for (int c = 0; c < 8; c++) load8<BF16>(w, row * K + col + 8 * c, v + 8 * c);
  } else {
#pragma unroll
    for (int i = 0; i < 64; i++) v[i] = 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; c++) m = __builtin_fmaxf(m, absmax8(v + 8 * c));
  m = group_max(m, 64);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  float s = m / 448.0f;
  if (s == 0.0f) s = 1.0f;
  const bool fast = s >= 0x1p-90f && s <= 0x1p90f;
  const float y = 1.0f / s;
  if (live) {
#pragma unroll
    for (int c = 0; c < 4; c++) {
      float q[16];
#pragma unroll
      for (int i = 0; i < 16; i++) q[i] = fast ? clamp448(div_rn_markstein(v[16 * c + i], s, y)) : clamp448(v[16 * c + i] / s);
      u32x4_t out;
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const uint32_t r = e4m3_pack2<false>(q[4 * d], q[4 * d + 1], 0u);
        out[d] = e4m3_pack2<true>(q[4 * d + 2], q[4 * d + 3], r);
      }
      *reinterpret_cast<u32x4_t*>(codes + row * K + col + 16 * c) = out;
    }
  }
  if (t == 0) scales[(int64_t)blockIdx.y * (K / 128) + blockIdx.x] = s;
}

// ---------------------------------------------------------------------------
// GEMM.  256 (weight rows) x 256 (activation rows) output tile per workgroup
// of 8 waves (2 along N x 4 along M, each 128 x 64), K step 128 = one scale
// block, two LDS stages of 32 KB per operand filled by direct-to-LDS loads one
// step ahead.  The weights are the MFMA's first operand, so a lane's 16x16
// output fragment holds one activation row and four consecutive channels of
// one 128-channel block: promoting a K block's partial sums takes one fp32
// factor per fragment.  v_mfma_scale_f32_16x16x128_f8f6f4 (neutral block
// scales) covers one K step per fragment.
// ---------------------------------------------------------------------------
constexpr int GBN = 256, GBM = 256, GBK = 128;
constexpr int GW_TILE = GBN * GBK;                       // 32 KB of E4M3 weight rows
constexpr int GX_TILE = GBM * GBK;                       // 32 KB of E4M3 activation rows
constexpr int GSTAGE = GW_TILE + GX_TILE;
constexpr int GLDS = 2 * GSTAGE;                         // 128 KB
// 128-byte rows: chunk c of row r sits at c ^ ((r >> 1) & 7).  The counters
// report LDS bank conflicts for the fragment reads (16 rows x 4 chunk pairs)
// with this placement and none with c ^ ((r ^ (r >> 3)) & 7), but the GEMM
// measured about 5 % faster with this one.
__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ i32x8_t ld_frag(const uint8_t* tile, int r, int q) {
  const u32x4_t p0 = ld16(tile + r * GBK + (((2 * q) ^ gswz(r)) << 4));
  const u32x4_t p1 = ld16(tile + r * GBK + (((2 * q + 1) ^ gswz(r)) << 4));
  return i32x8_t{(int)p0[0], (int)p0[1], (int)p0[2], (int)p0[3], (int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3]};
}

// PROMOTE: some scale depends on the K block; every block's partial sums are
// scaled and added to the accumulator.  Otherwise the scales go to the epilogue.
template <bool PROMOTE>
__global__ __launch_bounds__(512) void k_w8a8(const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
                                             int64_t as_m, int64_t as_k, const uint8_t* __restrict__ b,
                                             const float* __restrict__ b_scale, int64_t bs_n, int64_t bs_k,
                                             int group_n, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
                                             int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 2, wm = wave & 3;
  const int l16 = lane & 15, q = lane >> 4;

  const int nwg = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if (nwg % 8 == 0) pid = (pid % 8) * (nwg / 8) + pid / 8;
  const int tn = pid % tiles_n, tm = pid / tiles_n;
  const int64_t n0 = (int64_t)tn * GBN, m0 = (int64_t)tm * GBM;
  const int64_t nrows = N - n0 < GBN ? N - n0 : GBN;
  const int64_t mrows = M - m0 < GBM ? M - m0 : GBM;
  const auto rw = make_rsrc(b + n0 * K, nrows * K);
  const auto rx = make_rsrc(a + m0 * K, mrows * K);

  // DMA: per operand 32 instructions of 8 rows x 8 chunks; 4 per wave
  uint32_t off[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = 8 * (wave * 4 + i) + (lane >> 3);
    off[i] = (uint32_t)(r * K) + 16 * ((lane & 7) ^ gswz(r));
  }
  auto issue = [&](int stage, int64_t k0) {
    uint8_t* Wt = lds + stage * GSTAGE;
    uint8_t* Xt = Wt + GW_TILE;
#pragma unroll
    for (int i = 0; i < 4; i++) lds_dma16(rw, Wt + (wave * 4 + i) * 1024, off[i] + (uint32_t)k0);
#pragma unroll
    for (int i = 0; i < 4; i++) lds_dma16(rx, Xt + (wave * 4 + i) * 1024, off[i] + (uint32_t)k0);
  };

  // activation rows of this lane's four fragments (clamped: rows past M unused)
  int64_t mrow[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int64_t m = m0 + wm * 64 + 16 * j + l16;
    mrow[j] = m < M ? m : M - 1;
  }
  // this wave's 128-channel block (its rows never leave it; clamped to the
  // last block when all its rows are past N)
  const int64_t nblk = (n0 + wn * 128) / 128 < (N - 1) / 128 ? (n0 + wn * 128) / 128 : (N - 1) / 128;
  const bool bprom = PROMOTE && group_n == 128;

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)(K / GBK);
  float fa[4], fb = 1.0f, na[4], nb = 1.0f;             // scale factors of steps k and k + 1
  auto load_f = [&](int kt, float (&sa)[4], float& sb) {
#pragma unroll
    for (int j = 0; j < 4; j++) sa[j] = a_scale[mrow[j] * as_m + (int64_t)kt * as_k];
    sb = bprom ? b_scale[nblk * bs_n + (int64_t)kt * bs_k] : 1.0f;
  };
  issue(0, 0);
  if constexpr (PROMOTE) load_f(0, fa, fb);
  wait_vm<0>();
  tile_barrier();

  for (int kt = 0; kt < nk; kt++) {
    const int st = kt & 1;
    if (kt + 1 < nk) {
      issue(st ^ 1, (int64_t)(kt + 1) * GBK);
      if constexpr (PROMOTE) load_f(kt + 1, na, nb);
    }
    const uint8_t* Wt = lds + st * GSTAGE;
    const uint8_t* Xt = Wt + GW_TILE;
    i32x8_t bx[4];
#pragma unroll
    for (int j = 0; j < 4; j++) bx[j] = ld_frag(Xt, wm * 64 + 16 * j + l16, q);
    float f[4];
    if constexpr (PROMOTE) {
#pragma unroll
      for (int j = 0; j < 4; j++) f[j] = fa[j] * fb;
    }
    // weight fragment i + 1 is read while fragment i's MFMAs run
    i32x8_t awn = ld_frag(Wt, wn * 128 + l16, q);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const i32x8_t aw = awn;
      if (i < 7) awn = ld_frag(Wt, wn * 128 + 16 * (i + 1) + l16, q);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if constexpr (PROMOTE) {
          const f32x4_t t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, bx[j], f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                                             0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int r = 0; r < 4; r++) acc[i][j][r] = __builtin_fmaf(t[r], f[j], acc[i][j][r]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, bx[j], acc[i][j], 0, 0, 0, 127, 0, 127);
        }
      }
    }
    wait_vm<0>();
    tile_barrier();
    if constexpr (PROMOTE) {
#pragma unroll
      for (int j = 0; j < 4; j++) fa[j] = na[j];
      fb = nb;
    }
  }

  // epilogue: fragment element r sits at channel 4q + r, activation row l16.
  // Scales that do not depend on K multiply here.  Stores go through a buffer
  // range over the tile's rows below M; channels past N get an offset outside
  // the range.
  const auto ry = make_rsrc(y + m0 * N, mrows * N * 2);
  const bool vec = (N & 3) == 0;
  const int gsh = group_n == 128 ? 7 : 0;
  float sa[4];
#pragma unroll
  for (int j = 0; j < 4; j++) sa[j] = PROMOTE ? 1.0f : a_scale[mrow[j] * as_m];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int64_t nb0 = n0 + wn * 128 + 16 * i + 4 * q;
    float sb[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int64_t n = nb0 + r < N ? nb0 + r : N - 1;
      sb[r] = (!PROMOTE || group_n == 1) ? b_scale[(n >> gsh) * bs_n] : 1.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t rowoff = (uint32_t)((wm * 64 + 16 * j + l16) * N * 2);
      const uint32_t p01 = pack_bf16x2(acc[i][j][0] * (sa[j] * sb[0]), acc[i][j][1] * (sa[j] * sb[1]));
      const uint32_t p23 = pack_bf16x2(acc[i][j][2] * (sa[j] * sb[2]), acc[i][j][3] * (sa[j] * sb[3]));
      if (vec) {
        const uint32_t o = nb0 < N ? rowoff + (uint32_t)(nb0 * 2) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{p01, p23}, ry, (int)o, 0, 0);
      } else {
        const uint32_t pr[4] = {p01 & 0xFFFFu, p01 >> 16, p23 & 0xFFFFu, p23 >> 16};
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const uint32_t o = nb0 + r < N ? rowoff + (uint32_t)((nb0 + r) * 2) : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)pr[r], ry, (int)o, 0, 0);
        }
      }
    }
  }
}

template <auto KERNEL>
hipError_t allow_lds128() {
  static bool done[64] = {};
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && done[dev]) return hipSuccess;
  const hipError_t f =
      hipFuncSetAttribute(reinterpret_cast<const void*>(KERNEL), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (f == hipSuccess && dev >= 0 && dev < 64) done[dev] = true;
  return f;
}

}  // namespace

extern "C" {

wq_status quantize_e4m3_static(const void* x, int x_dtype, int64_t rows, int64_t cols, const float* scale,
                               uint8_t* codes, void* stream) {
  if (!x || !scale || !codes || rows <= 0 || cols <= 0 || cols % 16) return WQ_EINVAL;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16) return WQ_EUNSUPPORTED;
  if (!wq_numel_ok(rows, cols)) return WQ_EINVAL;
  if (!wq_aligned(x) || !wq_aligned(codes) || ((uintptr_t)scale & 3u)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nch = rows * cols / 16;
  if (x_dtype == WQ_BF16) k_e4m3_static<true><<<grid_for(nch), kThreads, 0, s>>>(x, nch, scale, codes);
  else k_e4m3_static<false><<<grid_for(nch), kThreads, 0, s>>>(x, nch, scale, codes);
  return wq_launch_status();
}

wq_status quantize_e4m3_block2d(const void* w, int w_dtype, int64_t rows, int64_t cols, uint8_t* codes, float* scales,
                                void* stream) {
  if (!w || !codes || !scales || rows <= 0 || cols <= 0 || cols % 128) return WQ_EINVAL;
  if (w_dtype != WQ_F32 && w_dtype != WQ_BF16) return WQ_EUNSUPPORTED;
  if (!wq_numel_ok(rows, cols) || (rows + 127) / 128 > 65535 || cols / 128 > 0x7FFFFFFF) return WQ_EINVAL;
  if (!wq_aligned(w) || !wq_aligned(codes) || ((uintptr_t)scales & 3u)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)(cols / 128), (unsigned)((rows + 127) / 128));
  if (w_dtype == WQ_BF16) k_e4m3_block2d<true><<<grid, kThreads, 0, s>>>(w, rows, cols, codes, scales);
  else k_e4m3_block2d<false><<<grid, kThreads, 0, s>>>(w, rows, cols, codes, scales);
  return wq_launch_status();
}

wq_status wq_gemm_w8a8(const uint8_t* a, const float* a_scale, int64_t as_m, int64_t as_k, const uint8_t* b,
                       const float* b_scale, int64_t bs_n, int64_t bs_k, int32_t group_n, int64_t M, int64_t N,
                       int64_t K, uint16_t* y, void* stream) {
  if (!a || !a_scale || !b || !b_scale || !y) return WQ_EINVAL;
  if (M <= 0 || N <= 0 || K <= 0 || K % GBK) return WQ_EINVAL;
  if (as_m < 0 || as_k < 0 || bs_n < 0 || bs_k < 0) return WQ_EINVAL;
  if (group_n != 1 && group_n != 128) return WQ_EUNSUPPORTED;
  if (group_n == 1 && bs_k != 0) return WQ_EUNSUPPORTED;        // per-channel scales do not depend on K
  if (!wq_numel_ok(M, K) || !wq_numel_ok(N, K) || !wq_numel_ok(M, N)) return WQ_EINVAL;
  // 32-bit buffer offsets: one 256-row tile of a, b and y
  if ((int64_t)GBN * K > 0x7FFFFFF0LL || (int64_t)GBM * N * 2 > 0x7FFFFFF0LL) return WQ_EINVAL;
  const int64_t tm = (M + GBM - 1) / GBM, tn = (N + GBN - 1) / GBN;
  if (tm * tn > 0x7FFFFFFF) return WQ_EINVAL;
  if (!wq_aligned(a) || !wq_aligned(b) || !wq_aligned(y)) return WQ_EALIGN;
  if (((uintptr_t)a_scale & 3u) || ((uintptr_t)b_scale & 3u)) return WQ_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = (unsigned)(tm * tn);
  if (as_k != 0 || bs_k != 0) {
    if (allow_lds128<k_w8a8<true>>() != hipSuccess) return WQ_EHIP;
    k_w8a8<true><<<grid, 512, GLDS, s>>>(a, a_scale, as_m, as_k, b, b_scale, bs_n, bs_k, group_n, M, N, K, y,
                                           (int)tm, (int)tn);
  } else {
    if (allow_lds128<k_w8a8<false>>() != hipSuccess) return WQ_EHIP;
    k_w8a8<false><<<grid, 512, GLDS, s>>>(a, a_scale, as_m, as_k, b, b_scale, bs_n, bs_k, group_n, M, N, K, y,
                                            (int)tm, (int)tn);
  }
  return wq_launch_status();
}

}  // extern "C"

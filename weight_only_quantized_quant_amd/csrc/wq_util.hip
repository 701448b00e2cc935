// Measurement utilities: a read-only streaming kernel (the measured HBM
// denominator of the decode GEMV) and a bounded busy kernel that keeps the
// device occupied while a timed region is submitted.
#include <hip/hip_runtime.h>

#include "wq_device.h"
#include "wq_host.h"
#include "wq_util.h"

using namespace wq;

namespace {

constexpr int SR_THREADS = 256, SR_LOADS = 8;
constexpr int64_t SR_PIECE = (int64_t)SR_THREADS * SR_LOADS * 16;     // 32 KB per workgroup

// Workgroup b reads bytes [b * 32 KB, (b + 1) * 32 KB) of the buffer: load u
// of lane t at byte (u * 256 + t) * 16, so each wave instruction reads 1 KB
// contiguously.  The buffer resource ends at the buffer's end, so the last
// piece's loads past it return zeros without touching memory.
__global__ __launch_bounds__(SR_THREADS) void k_stream_read(const uint8_t* __restrict__ buf, int64_t bytes,
                                                            uint32_t magic, uint32_t* __restrict__ sink) {
  const int64_t off = (int64_t)blockIdx.x * SR_PIECE;
  const int64_t left = bytes - off;
  const auto r = make_rsrc(buf + off, left < SR_PIECE ? left : SR_PIECE);
  u32x4_t v[SR_LOADS];
#pragma unroll
  for (int u = 0; u < SR_LOADS; u++) v[u] = bld16(r, (uint32_t)(u * SR_THREADS + threadIdx.x) * 16);
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < SR_LOADS; u++) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (acc == magic) sink[0] = acc;
}

__global__ __launch_bounds__(256) void k_spin(int64_t iters, uint32_t magic, uint32_t* __restrict__ sink) {
  float a = (float)threadIdx.x, b = a + 1.0f, c = a + 2.0f, d = a + 3.0f;
  for (int64_t i = 0; i < iters; i++) {
    a = __builtin_fmaf(a, 0.999f, 0.5f);
    b = __builtin_fmaf(b, 0.999f, 0.5f);
    c = __builtin_fmaf(c, 0.999f, 0.5f);
    d = __builtin_fmaf(d, 0.999f, 0.5f);
  }
  if ((__float_as_uint(a) ^ __float_as_uint(b) ^ __float_as_uint(c) ^ __float_as_uint(d)) == magic) sink[0] = magic;
}

// One wave stamps the shader cycle counter (s_memtime) and the constant-rate
// wall clock (s_memrealtime) at its start, polls the wall clock until `ticks`
// ticks have passed (at most 2^20 polls), stamps both again and stores the
// two differences: their ratio times the wall clock's rate is the shader
// clock over that interval.
__global__ __launch_bounds__(64) void k_clock(int64_t ticks, int64_t* __restrict__ out) {
  const int64_t c0 = (int64_t)__builtin_amdgcn_s_memtime(), w0 = (int64_t)__builtin_amdgcn_s_memrealtime();
  int64_t w = w0;
  for (int i = 0; i < (1 << 20) && w - w0 < ticks; i++) w = (int64_t)__builtin_amdgcn_s_memrealtime();
  const int64_t c1 = (int64_t)__builtin_amdgcn_s_memtime(), w1 = (int64_t)__builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = w1 - w0;
  }
}

}  // namespace

extern "C" {

wq_status wq_util_stream_read(const void* buf, int64_t bytes, uint32_t magic, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || bytes > (int64_t(1) << 40)) return WQ_EINVAL;
  if (!wq_aligned(buf)) return WQ_EALIGN;
  const int64_t grid = (bytes + SR_PIECE - 1) / SR_PIECE;
  k_stream_read<<<(unsigned)grid, SR_THREADS, 0, (hipStream_t)stream>>>((const uint8_t*)buf, bytes, magic, sink);
  return wq_launch_status();
}

wq_status wq_util_spin(int64_t iters, uint32_t magic, uint32_t* sink, void* stream) {
  if (!sink || iters < 1 || iters > (int64_t(1) << 24)) return WQ_EINVAL;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    return WQ_EHIP;
  k_spin<<<(unsigned)ncu, 256, 0, (hipStream_t)stream>>>(iters, magic, sink);
  return wq_launch_status();
}

wq_status wq_util_clock(int64_t ticks, int64_t* out, void* stream) {
  if (!out || ticks < 1 || ticks > (int64_t(1) << 20)) return WQ_EINVAL;
  if (!wq_aligned(out)) return WQ_EALIGN;
  k_clock<<<1, 64, 0, (hipStream_t)stream>>>(ticks, out);
  return wq_launch_status();
}

wq_status wq_util_wall_clock_khz(int* khz) {
  int dev = 0;
  if (!khz) return WQ_EINVAL;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      *khz <= 0)
    return WQ_EHIP;
  return WQ_OK;
}

}  // extern "C"

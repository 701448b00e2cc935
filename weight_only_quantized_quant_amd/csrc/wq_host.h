// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq.h"

inline bool wq_aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// rows * cols within 2^40 elements (index arithmetic stays in int64).
inline bool wq_numel_ok(int64_t rows, int64_t cols) {
  return rows > 0 && cols > 0 && rows <= (int64_t(1) << 40) / cols;
}

inline wq_status wq_launch_status() {
  return hipGetLastError() == hipSuccess ? WQ_OK : WQ_EHIP;
}

/*
 * wq_util.h -- measurement utilities of libwq.so.
 *
 * They are not steps of the quantization path: they exist so that a
 * benchmark can put a measured denominator beside the kernels' timings and
 * keep launch latency out of a timed region.  Same conventions as wq.h:
 * caller-owned device pointers, asynchronous work on `stream` (a hipStream_t,
 * NULL = default stream), host-side validation, wq_status results.
 */
#ifndef WQ_UTIL_H
#define WQ_UTIL_H

#include <stddef.h>
#include <stdint.h>

#include "wq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * wq_util_stream_read -- read `bytes` bytes of device memory once, front to
 * back, with 16-byte loads (each workgroup of 256 lanes reads one contiguous
 * 32 KB piece, eight loads per lane in flight), and discard them.
 *
 * The roofline of the weight-only matmul in decode is the time to stream the
 * packed weights from HBM once ("Numerics: FP32 to INT4, and why bf16 won",
 * bytes per parameter times parameters over bandwidth); this kernel measures
 * that time on the machine for a given footprint.
 *
 * buf    device buffer of `bytes` bytes, 16-byte aligned (WQ_EALIGN).
 * bytes  > 0, a multiple of 16, at most 2^40 (WQ_EINVAL).
 * sink   one device uint32.  A lane writes the XOR of what it read there only
 *        when that XOR equals `magic` (so that no read can be optimised
 *        away); its contents are meaningless.
 */
wq_status wq_util_stream_read(const void* buf, int64_t bytes, uint32_t magic, uint32_t* sink, void* stream);

/*
 * wq_util_spin -- a bounded busy kernel: one workgroup of 256 lanes per
 * compute unit runs `iters` iterations of four dependent fp32 fma chains and
 * exits.  There is no flag or other input that could keep it running: its
 * duration is fixed by `iters` (about 16 shader cycles per iteration).
 *
 * Enqueued ahead of a timed region, it keeps the device busy while the host
 * submits the region's launches, so that the submission latency of the
 * region stays off the clock.
 *
 * iters  1 .. 2^24 (WQ_EINVAL otherwise).
 * sink   one device uint32, written only when the chains end on `magic`; its
 *        contents are meaningless.
 */
wq_status wq_util_spin(int64_t iters, uint32_t magic, uint32_t* sink, void* stream);

/*
 * wq_util_clock -- one wave records the shader clock over a short interval:
 * it reads the shader cycle counter and the constant-rate wall clock, polls
 * the wall clock until `ticks` ticks have passed (or 2^20 polls, whichever
 * comes first), reads both again and stores out[0] = cycles elapsed and
 * out[1] = wall ticks elapsed.  The shader clock over the interval is
 * out[0] / out[1] times the wall clock's rate (wq_util_wall_clock_khz).
 *
 * Enqueued just before and just after a timed region on the same stream, it
 * records the clock that the region ran at (a clock set by power management
 * changes over milliseconds; the region lasts a fraction of one).
 *
 * ticks  1 .. 2^20 wall-clock ticks (WQ_EINVAL otherwise).
 * out    two device int64, 16-byte aligned (WQ_EALIGN), written by the kernel.
 */
wq_status wq_util_clock(int64_t ticks, int64_t* out, void* stream);

/* wq_util_wall_clock_khz -- rate of the current device's wall clock (the
 * counter wq_util_clock reads as out[1]) in kHz, written to *khz. */
wq_status wq_util_wall_clock_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* WQ_UTIL_H */

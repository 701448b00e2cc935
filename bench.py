"""Benchmark of the weight-only quantized matmul and the block-scaled quantizers
on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only CASE] [--no-cpu]

One step is one decode GEMV y = x . dequant(Wq)^T at M = 1, K = 4096,
N = 14336 with symmetric INT4 weights (bf16 scales per 128-element group),
bf16 activations and output -- the decode W4A16 workload.  The weights are
quantized on the GPU by quantize_int4 and replicated into 24 resident copies
(727 MB) that the steps cycle through, so that the 256 MB Infinity Cache
cannot serve them: every step streams its weights from HBM.  The K timed
steps are launched as one HIP graph replay behind a bounded busy kernel (so
that the host's submission stays off the clock; see Region), in --rounds
rounds; ms per step is the median round and `value` is algorithmic bytes /
that time.

The same JSON line carries the roofline of that kernel (HIP events over the
timed region on the launch stream), the oracle timed on the host (`cpu_baseline`)
and `secondary` measurements: decode at M = 4 and 16, W8A16, asymmetric INT4
decode at M = 1, NVFP4 decode at M = 1 and 16, prefill MXFP4 and NVFP4 at M = 8192 (TFLOP/s), the activation
quantizers at 4096 x 7168 (E4M3 per 128, MXFP4 per 16, MXFP8 per 32 under two
E8M0 rules, and the share of blocks whose maximum clips under each rule), the
MXFP4 weight quantizer, the W8A8 FP8 GEMM at the prefill shape (block-scaled
and per-token x per-channel), the W4A8 mixture-of-experts grouped GEMMs (gate/up and
down, with routing, token quantization and prepack), a streaming copy and
torch.matmul (hipBLASLt) at the prefill shape as secondary denominators.
`gpu_clocks_hwmon` holds SCLK, MCLK and board power sampled from the GPU's
sysfs files during the decode timed region and the prefill timed rounds (left
out where sysfs does not expose them).

--only CASE runs a single case without the full summary (for rocprofv3):
decode (the same graph-timed steps as the headline, prints one short JSON
line), decode_m1 (the headline's launches, eager, for counter runs), decode_m4, decode_m16, decode_w8, decode_nvfp4, decode_asym, prefill, prefill_nvfp4, prefill_int4, w8a8_block, w8a8_channel, quant_e4m3, quant_mxfp4, quant_mxfp8, wquant_mxfp4, copy,
moe_gate_up, moe_down, stream_decode (the read-only stream of the decode weight
copies), stream_2g, torch_matmul (hipBLASLt on the dequantized prefill weights).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
ROTATE_BYTES = 700e6           # > 2.5x the 256 MB Infinity Cache
DECODE_KERNEL = "k_gemv_ring<INT4> (wq_gemm, M<=4 decode path)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--only", default=None)
    p.add_argument("--reps", type=int, default=0, help="launches for --only (default per case)")
    p.add_argument("--rounds", type=int, default=5, help="timed regions of --steps launches (median)")
    p.add_argument("--no-cpu", action="store_true")
    return p.parse_args()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def graph_of(torch, fns):
    """Capture the callables (each enqueues one launch) into one HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fns[0]()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, launches):
    """HIP events on the current stream around one replay; ms per launch
    (secondary measurements; the headline uses time_region)."""
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    b.synchronize()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / launches


class Region:
    """Timed regions of exactly `launches` launches, each preceded by a bounded
    busy kernel (wq_util_spin) on the same stream, so that the host submits the
    region's launches while the device is still busy and the submission
    latency stays off the clock: event a fires when the busy kernel ends, and
    the first launch follows at once.  The busy kernel's iteration count is
    sized from a measured rate to last about eight times the host's submission
    time (at least 0.3 ms): the submission time of one region varies with the
    host's load, and a region whose launches are still being submitted when
    the busy kernel ends is timed partly on the host.
    `rounds` regions are timed; ms per launch is their median.  A one-wave
    clock probe (wq_util_clock) runs just before event a and just after event
    b and records the shader clock at each end of every region."""

    def __init__(self, torch, W, enqueue, launches, rounds=5):
        self.torch, self.W, self.enqueue, self.launches, self.rounds = torch, W, enqueue, launches, rounds
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        W.wq_util_spin(20000)
        b.record()
        b.synchronize()
        self.ms_per_iter = max(a.elapsed_time(b) / 20000, 1e-6)
        t = time.perf_counter()
        enqueue()                                   # untimed pass: host submission time
        self.host_ms = (time.perf_counter() - t) * 1e3
        torch.cuda.synchronize()
        self.iters = int(min(max(max(8.0 * self.host_ms, 0.3) / self.ms_per_iter, 1000), 1 << 24))
        self.windows = []
        self.clk = torch.zeros((rounds, 2, 2), dtype=torch.int64, device="cuda")
        self.wall_khz = W.wq_util_wall_clock_khz()

    def run(self, sampler=None):
        torch = self.torch
        ms, covered = [], []
        for r in range(self.rounds):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            self.W.wq_util_spin(self.iters)
            self.W.wq_util_clock(self.clk[r, 0])
            a.record()
            self.enqueue()
            b.record()
            self.W.wq_util_clock(self.clk[r, 1])
            t1 = time.perf_counter()
            b.synchronize()
            t2 = time.perf_counter()
            ms.append(a.elapsed_time(b) / self.launches)
            # the busy kernel outlasted the submission when the host was done
            # before the busy kernel's planned end
            covered.append((t1 - t0) * 1e3 < self.iters * self.ms_per_iter)
            self.windows.append((t0, t2))
        self.ms_rounds = ms
        self.covered = all(covered)
        c = self.clk.cpu().numpy().astype(np.float64)
        self.mhz = c[:, :, 0] / np.maximum(c[:, :, 1], 1) * self.wall_khz * 1e-3
        return float(np.median(ms))

    def describe(self):
        return {"rounds_us_per_launch": [round(m * 1e3, 3) for m in self.ms_rounds],
                "median_of_rounds": len(self.ms_rounds), "launches_per_round": self.launches,
                "busy_kernel_us": round(self.iters * self.ms_per_iter * 1e3, 1),
                "host_submit_us": round(self.host_ms * 1e3, 1), "busy_kernel_covered_submission": self.covered,
                "shader_clock_mhz": {"before_region": [round(v) for v in self.mhz[:, 0]],
                                     "after_region": [round(v) for v in self.mhz[:, 1]]}}


class ClockSampler:
    """SCLK, MCLK and board power of the GPU, read from its sysfs files (hwmon,
    else the current level of pp_dpm_sclk / pp_dpm_mclk) on a background
    thread while a timed region runs.  Keys whose files are missing or
    unreadable are left out."""

    FILES = (("sclk_mhz", "freq1_input", 1e-6), ("mclk_mhz", "freq2_input", 1e-6),     # Hz, microwatts
             ("power_w", "power1_average", 1e-6), ("power_w", "power1_input", 1e-6))

    def __init__(self, torch):
        import threading
        self.files, self.samples, self.stamped = {}, {}, {}
        self.stop_evt, self.thread = threading.Event(), None
        try:
            p = torch.cuda.get_device_properties(0)
            dev = f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
            for h in sorted(os.listdir(os.path.join(dev, "hwmon"))):
                for key, fn, scale in self.FILES:
                    f = os.path.join(dev, "hwmon", h, fn)
                    if key not in self.files and os.access(f, os.R_OK):
                        self.files[key] = (f, scale)
            for key, fn in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
                f = os.path.join(dev, fn)
                if key not in self.files and os.access(f, os.R_OK):
                    self.files[key] = (f, None)
        except (OSError, AttributeError):
            pass

    @staticmethod
    def _value(text, scale):
        if scale is not None:
            return int(text.strip()) * scale
        for line in text.splitlines():                  # "1: 2400Mhz *" marks the current level
            if line.rstrip().endswith("*"):
                return float(line.split(":")[1].strip().split()[0].lower().replace("mhz", ""))
        raise ValueError("no current level")

    def _run(self):
        while not self.stop_evt.is_set():
            for key, (f, scale) in self.files.items():
                try:
                    with open(f) as fh:
                        v = self._value(fh.read(), scale)
                    self.samples.setdefault(key, []).append(v)
                    self.stamped.setdefault(key, []).append((time.perf_counter(), v))
                except (OSError, ValueError, IndexError):
                    pass
            self.stop_evt.wait(0.00025)

    def __enter__(self):
        import threading
        self.samples, self.stamped = {}, {}
        self.stop_evt.clear()
        if self.files:
            self.thread = threading.Thread(target=self._run, daemon=True)
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop_evt.set()
        if self.thread is not None:
            self.thread.join()
            self.thread = None
        return False

    def summary(self):
        return {k: {"median": round(float(np.median(v)), 1), "min": round(float(np.min(v)), 1),
                    "max": round(float(np.max(v)), 1), "samples": len(v)}
                for k, v in self.samples.items() if v} or None

    def per_window(self, windows):
        """Samples taken inside each (t0, t1) host window, per key."""
        out = []
        for t0, t1 in windows:
            out.append({k: [round(v, 1) for t, v in sv if t0 <= t <= t1] for k, sv in self.stamped.items()})
        return out


def time_eager(torch, fn, reps, warm=3, rounds=3):
    """Median over `rounds` timed rounds of `reps` eager launches, after `warm`
    untimed launches (the first launches of a large kernel run before the
    clocks have settled)."""
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    ms = []
    for _ in range(rounds):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            fn(i)
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b) / reps)
    return sorted(ms)[len(ms) // 2]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("csrc/wq_gemm.hip", "csrc/wq_device.h", "csrc/wq_quant.hip", "build.py"):
        with open(os.path.join(ROOT, "weight_only_quantized_quant_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(case, bytes_per_launch):
    """HBM traffic from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(case)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def nvfp4_tensor_scale(torch, w):
    """Per-tensor scale that maps the tensor's maximum to 6 * 448."""
    return float(w.abs().max().item()) / (6.0 * 448.0)


def packed_copy(torch, parts):
    """One device byte buffer holding `parts` (contiguous tensors) back to back,
    each at a 256-byte boundary; returns (buffer, views of the parts, bytes
    used).  The weight copies of a decode workload live in such buffers, so
    that one streaming read covers exactly their footprint."""
    offs, o = [], 0
    for t in parts:
        offs.append(o)
        o += (t.numel() * t.element_size() + 255) // 256 * 256
    buf = torch.empty(o, dtype=torch.uint8, device="cuda")
    views = []
    for t, off in zip(parts, offs):
        n = t.numel() * t.element_size()
        v = buf[off:off + n].view(t.dtype).view(t.shape)
        v.copy_(t)
        views.append(v)
    return buf, views, o


class Decode:
    """x[M, 4096] . dequant(W[14336, 4096])^T, INT4 g128 (symmetric, or
    asymmetric with a zero-point), E4M3 per-channel or NVFP4 (E4M3 scale per
    16, per-tensor fp32 scale).  Each weight copy (codes, then scales) lives in
    one buffer; the copies together exceed the 256 MB Infinity Cache."""

    def __init__(self, torch, W, M, kind="int4", K=4096, N=14336):
        from synthetic import decode_inputs
        self.torch, self.W, self.M, self.K, self.N, self.kind = torch, W, M, K, N, kind
        xbits, Wf = decode_inputs(M, seed=0)
        self.x = dev_bf16(torch, xbits)
        wdev = torch.from_numpy(Wf).cuda()
        self.alpha = 1.0
        if kind == "int4":
            packed, sb = W.quantize_int4(wdev, 128)
            self.wbytes = packed.numel() * 4 + sb.numel() * 2
            base = (packed, sb)
            self.meta = (W.WQ_INT4X8, W.WQ_BF16, 128)
        elif kind == "int4_asym":
            packed, sz = W.quantize_int4_asym(wdev, 128)
            self.wbytes = packed.numel() * 4 + sz.numel() * 4
            base = (packed, sz)
            self.meta = (W.WQ_UINT4X8, W.WQ_BF16Z, 128)
        elif kind == "nvfp4":
            self.alpha = nvfp4_tensor_scale(torch, wdev)
            codes, sc = W.quantize_nvfp4(wdev, self.alpha)
            self.wbytes = codes.numel() + sc.numel()
            base = (codes, sc)
            self.meta = (W.WQ_E2M1X2, W.WQ_E4M3, 16)
        else:
            codes, sc = W.quantize_e4m3(wdev, -1)
            sc = sc.reshape(-1).contiguous()
            self.wbytes = codes.numel() + sc.numel() * 4
            base = (codes, sc)
            self.meta = (W.WQ_E4M3, W.WQ_F32, K)
        del wdev
        ncopy = max(1, int(ROTATE_BYTES // self.wbytes) + 1)
        self.bufs, self.copies = [], []
        for _ in range(ncopy):
            buf, views, _ = packed_copy(torch, base)
            self.bufs.append(buf)
            self.copies.append(tuple(views))
        del base
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        self.bytes = self.wbytes + M * K * 2 + M * N * 2
        self.flops = 2.0 * M * N * K

    def launch(self, i):
        wq, sc = self.copies[i % len(self.copies)]
        wdt, sdt, grp = self.meta
        self.W.wq_gemm(self.x, wq, wdt, sc, sdt, grp, self.N, y=self.y, alpha=self.alpha)

    def stream(self, i):
        """Read-only stream of copy i's weights and scales (the footprint the
        GEMV must read from HBM, x and y aside)."""
        self.W.wq_util_stream_read(self.bufs[i % len(self.bufs)])


class BigStream:
    """Read-only stream of a 2 GiB buffer (the steady-state HBM read rate)."""

    def __init__(self, torch, W, nbytes=2 << 30):
        self.W = W
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        self.bytes = nbytes

    def launch(self, i):
        self.W.wq_util_stream_read(self.buf)


class Prefill:
    """x[8192, 4096] . dequant(W[14336, 4096])^T with MXFP4 (E8M0 per 32),
    NVFP4 (E4M3 per 16 and a per-tensor scale) or symmetric INT4 (bf16 scale
    per 128) weights."""

    def __init__(self, torch, W, M=8192, K=4096, N=14336, kind="mxfp4"):
        from synthetic import prefill_inputs
        self.torch, self.W, self.M, self.K, self.N, self.kind = torch, W, M, K, N, kind
        xbits, Wf = prefill_inputs(0, M=M, K=K, N=N)
        self.x = dev_bf16(torch, xbits)
        wdev = torch.from_numpy(Wf).cuda()
        if kind == "nvfp4":
            self.alpha = nvfp4_tensor_scale(torch, wdev)
            self.codes, self.sc = W.quantize_nvfp4(wdev, self.alpha)
            self.meta = (W.WQ_E2M1X2, W.WQ_E4M3, 16)
        elif kind == "int4":
            self.alpha = 1.0
            packed, self.sc = W.quantize_int4(wdev, 128)
            self.codes = packed.view(torch.uint8)
            self.meta = (W.WQ_INT4X8, W.WQ_BF16, 128)
        else:
            self.alpha = 1.0
            self.codes, self.sc = W.quantize_mxfp4(wdev, 32)
            self.meta = (W.WQ_E2M1X2, W.WQ_E8M0, 32)
        del wdev
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        self.flops = 2.0 * M * N * K
        self.bytes = (self.codes.numel() * self.codes.element_size() + self.sc.numel() * self.sc.element_size()
                      + M * K * 2 + M * N * 2)

    def launch(self, i):
        wdt, sdt, grp = self.meta
        self.W.wq_gemm(self.x, self.codes, wdt, self.sc, sdt, grp, self.N, y=self.y, alpha=self.alpha)


class W8A8:
    """x[8192, 4096] . W[14336, 4096]^T in W8A8 FP8: "block" = per-token
    1x128-group activation scales and 128x128 weight blocks (scales folded in
    per K block); "channel" = per-token activation and per-channel weight
    scales (applied to the finished sums).  Quantized on the GPU."""

    def __init__(self, torch, W, mode, M=8192, K=4096, N=14336):
        from synthetic import prefill_inputs
        self.W, self.M, self.K, self.N, self.mode = W, M, K, N, mode
        xbits, Wf = prefill_inputs(0, M=M, K=K, N=N)
        x = dev_bf16(torch, xbits)
        wdev = torch.from_numpy(Wf).cuda()
        if mode == "block":
            self.a, sa = W.quantize_e4m3(x, 128)
            self.b, sb = W.quantize_e4m3_block2d(wdev)
            self.args = (sa.reshape(-1), K // 128, 1, sb.reshape(-1), K // 128, 1, 128)
        else:
            self.a, sa = W.quantize_e4m3(x, -1)
            self.b, sb = W.quantize_e4m3(wdev, -1)
            self.args = (sa.reshape(-1), 1, 0, sb.reshape(-1), 1, 0, 1)
        del wdev, x
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        self.flops = 2.0 * M * N * K

    def launch(self, i):
        sa, as_m, as_k, sb, bs_n, bs_k, gn = self.args
        self.W.wq_gemm_w8a8(self.a, sa, as_m, as_k, self.b, sb, bs_n, bs_k, gn, y=self.y)


class ActQuant:
    """4096 x 7168 bf16 -> E4M3 per 1x128 (fp32 scales), MXFP4 per 16 (E8M0) or
    MXFP8 (E4M3 elements, E8M0 per 32) under a chosen scale rule."""

    def __init__(self, torch, W, kind, rule="round"):
        from synthetic import act_quant_inputs
        self.torch, self.W, self.kind, self.rule = torch, W, kind, rule
        bits = act_quant_inputs(0)
        x = dev_bf16(torch, bits)
        rows, cols = bits.shape
        inb = rows * cols * 2
        if kind == "e4m3":
            shapes = ((rows, cols), torch.uint8), ((rows, cols // 128), torch.float32)
        elif kind == "mxfp4":
            shapes = ((rows, cols // 2), torch.uint8), ((rows, cols // 16), torch.uint8)
        else:
            shapes = ((rows, cols), torch.uint8), ((rows, cols // 32), torch.uint8)
        outb = sum(a * b * (4 if dt == torch.float32 else 1) for (a, b), dt in shapes)
        self.bytes = inb + outb
        ncopy = max(1, int(ROTATE_BYTES // self.bytes) + 1)
        self.xs = [x] + [x.clone() for _ in range(ncopy - 1)]
        self.outs = [tuple(torch.empty(sh, dtype=dt, device="cuda") for sh, dt in shapes) for _ in range(ncopy)]

    def launch(self, i):
        j = i % len(self.xs)
        c, s = self.outs[j]
        if self.kind == "e4m3":
            self.W.quantize_e4m3(self.xs[j], 128, codes=c, scales=s)
        elif self.kind == "mxfp4":
            self.W.quantize_mxfp4(self.xs[j], 16, codes=c, scales=s)
        else:
            self.W.quantize_mx(self.xs[j], 32, "e4m3", self.rule, codes=c, scales=s)


def clip_share(torch, W, x, block, elem, rule):
    """Share of blocks whose maximum lands above the element maximum (it then
    saturates) under `rule`, from the GPU scales of one quantize_mx call."""
    _, sc = W.quantize_mx(x, block, elem, rule)
    amax = x.float().abs().view(x.shape[0], -1, block).amax(dim=2)
    ratio = amax / torch.exp2(sc.float() - 127.0)
    return round(float((ratio > (6.0 if elem == "e2m1" else 448.0)).float().mean()), 5)


class WeightQuant:
    """14336 x 4096 fp32 -> MXFP4 block 32 (offline weight preparation)."""

    def __init__(self, torch, W):
        from synthetic import prefill_inputs
        self.W = W
        _, Wf = prefill_inputs(0, with_x=False)
        self.w = [torch.from_numpy(Wf).cuda()]
        self.w.append(self.w[0].clone())
        rows, cols = Wf.shape
        self.bytes = rows * cols * 4 + rows * cols // 2 + rows * cols // 32
        self.outs = [(torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
                      torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")) for _ in range(2)]

    def launch(self, i):
        c, s = self.outs[i % 2]
        self.W.quantize_mxfp4(self.w[i % 2], 32, codes=c, scales=s)


class MoeW4A8:
    """W4A8 mixture-of-experts grouped GEMM: 64 experts, top-8 routing of 4096
    tokens, hidden 4096, expert intermediate 1536.  which = "gate_up" (rows
    gathered by token, N = 3072, K = 4096) or "down" (grouped rows, N = 4096,
    K = 1536).  INT4 group-128 weights quantized on the GPU from device-side
    N(0, 0.02) weights, then prepacked; per-token E4M3 activations."""

    def __init__(self, torch, W, which):
        from synthetic import moe_down_input_gpu, moe_expert_weight_gpu, moe_router_logits, moe_tokens
        E, T, k, inter, hidden = 64, 4096, 8, 1536, 4096
        self.W, self.which = W, which
        self.N, self.K = (2 * inter, hidden) if which == "gate_up" else (hidden, inter)
        self.logits = torch.from_numpy(moe_router_logits(0)).cuda()
        _, _, self.off, rt, _ = W.wq_moe_route(self.logits, k)
        if which == "gate_up":
            self.x = dev_bf16(torch, moe_tokens())
            self.rt = rt
        else:
            self.x = moe_down_input_gpu(rows=T * k, inter=inter)
            self.rt = None
        self.x8, a = W.quantize_e4m3(self.x, -1)
        self.a = a.reshape(-1).contiguous()
        self.packed = torch.empty((E, self.N, self.K // 8), dtype=torch.int32, device="cuda")
        self.sb = torch.empty((E, self.N, self.K // 128), dtype=torch.bfloat16, device="cuda")
        for e in range(E):
            W.quantize_int4(moe_expert_weight_gpu(e, which, hidden=hidden, inter=inter), 128,
                            packed=self.packed[e], scales=self.sb[e])
        self.wq, self.s8, self.ch = W.wq_w4a8_prepack(self.packed, self.sb)
        self.R = T * k
        self.y = torch.empty((self.R, self.N), dtype=torch.bfloat16, device="cuda")
        self.flops = 2.0 * self.R * self.N * self.K
        self.k = k

    def launch(self, i):
        self.W.wq_moe_gemm_w4a8(self.x8, self.a, self.rt, self.off, self.wq, self.s8, self.ch, y=self.y)


class TorchMatmul:
    """torch.matmul (hipBLASLt) of the prefill activations with the dequantized
    MXFP4 weights of the prefill workload (the bf16 GEMM the kernel is
    compared with)."""

    def __init__(self, torch, W):
        pf = Prefill(torch, W)
        self.torch, self.x = torch, pf.x
        self.wb = W.wq_dequant(pf.codes, W.WQ_E2M1X2, pf.sc, W.WQ_E8M0, 32, pf.N, pf.K)
        self.flops = pf.flops
        del pf

    def launch(self, i):
        self.torch.matmul(self.x, self.wb.t())


class Copy:
    """Streaming copy of 256 MiB (read + write) as a secondary HBM denominator."""

    def __init__(self, torch):
        n = 1 << 26
        self.a = [torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0) for _ in range(3)]
        self.b = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
        self.bytes = 2 * n * 4

    def launch(self, i):
        self.b[i % 3].copy_(self.a[i % 3])


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the decode workload
# ---------------------------------------------------------------------------

def cpu_baseline(rows=14336, reps=3):
    from threadpoolctl import threadpool_limits
    from oracle import dequant as OD
    from oracle import gemm as OG
    from oracle import int4 as OI
    from synthetic import decode_inputs
    xbits, Wf = decode_inputs(1, seed=0)
    Wf = Wf[:rows]
    packed, sb, _ = OI.quantize_int4(Wf, 128)          # weight preparation, not timed
    K = Wf.shape[1]
    nbytes = packed.nbytes + sb.nbytes + K * 2 + rows * 2
    ncores = len(os.sched_getaffinity(0))

    def timed(threads):
        times = []
        with threadpool_limits(limits=threads):
            for _ in range(reps):
                t = time.perf_counter()
                wd = OD.dequant_int4(packed, sb, 128)
                OG.reference(xbits, wd)
                times.append(time.perf_counter() - t)
        return float(np.median(times))

    t1 = timed(1)
    tn = timed(ncores)
    # the reported figure is the faster of the two thread counts
    best, cores = (tn, ncores) if tn < t1 else (t1, 1)
    return {"value": nbytes / best / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"decode W4A16 M=1 K=4096 on {rows} of the 14336 output rows "
                      f"(INT4 dequant in NumPy, fp64 matvec through BLAS), median of {reps}; BLAS threads 1 and "
                      f"{ncores} (all cores in the affinity mask) both timed",
            "seconds_per_sample_step": best,
            "by_threads": {"1": {"GB/s": nbytes / t1 / 1e9, "s": t1},
                           str(ncores): {"GB/s": nbytes / tn / 1e9, "s": tn}},
            "os_cpu_count": os.cpu_count(), "affinity_cores": ncores}


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(no collective or sharded path is built).", file=sys.stderr)
        sys.exit(2)
    import torch
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    K, Wm = args.steps, args.warmup
    if args.only and args.only != "decode":
        case = args.only
        mk = {"decode_w8": lambda: Decode(torch, W, 1, "e4m3"), "decode_nvfp4": lambda: Decode(torch, W, 1, "nvfp4"),
              "decode_m1": lambda: Decode(torch, W, 1),
              "decode_m16": lambda: Decode(torch, W, 16), "decode_m4": lambda: Decode(torch, W, 4),
              "decode_asym": lambda: Decode(torch, W, 1, "int4_asym"),
              "prefill_nvfp4": lambda: Prefill(torch, W, kind="nvfp4"),
              "prefill_int4": lambda: Prefill(torch, W, kind="int4"),
              "w8a8_block": lambda: W8A8(torch, W, "block"), "w8a8_channel": lambda: W8A8(torch, W, "channel"),
              "prefill": lambda: Prefill(torch, W), "quant_e4m3": lambda: ActQuant(torch, W, "e4m3"),
              "quant_mxfp4": lambda: ActQuant(torch, W, "mxfp4"), "copy": lambda: Copy(torch),
              "quant_mxfp8": lambda: ActQuant(torch, W, "mxfp8"),
              "wquant_mxfp4": lambda: WeightQuant(torch, W),
              "moe_gate_up": lambda: MoeW4A8(torch, W, "gate_up"), "moe_down": lambda: MoeW4A8(torch, W, "down"),
              "stream_decode": lambda: Decode(torch, W, 1), "stream_2g": lambda: BigStream(torch, W),
              "torch_matmul": lambda: TorchMatmul(torch, W)}[case]
        obj = mk()
        big = case in ("prefill", "prefill_nvfp4", "prefill_int4", "moe_gate_up", "moe_down", "w8a8_block", "w8a8_channel",
                       "torch_matmul")
        reps = args.reps or (20 if big else 100)
        # the clocks settle over the first launches of a large kernel: the
        # profile's median then reflects the steady state, as the timed runs do
        fn = obj.stream if case == "stream_decode" else obj.launch
        for i in range(reps + (3 if big else 0)):
            fn(i)
        torch.cuda.synchronize()
        print(f"{case}: {reps} launches done", flush=True)
        return

    dec = Decode(torch, W, 1)
    warm_g = graph_of(torch, [lambda i=i: dec.launch(i) for i in range(max(1, Wm))])
    timed_g = graph_of(torch, [lambda i=i: dec.launch(i) for i in range(K)])
    warm_g.replay()
    torch.cuda.synchronize()
    region = Region(torch, W, timed_g.replay, K, rounds=args.rounds)
    clocks = ClockSampler(torch)
    t0 = time.perf_counter()
    with clocks:
        ms = region.run()
    wall = time.perf_counter() - t0
    clock_summary = {"decode_timed_regions": clocks.summary(),
                     "decode_per_region": clocks.per_window(region.windows)}
    value = dec.bytes / (ms * 1e-3) / 1e9
    # the measured denominator: a read-only stream of the same weight copies,
    # same rotation, same timing method
    stream_g = graph_of(torch, [lambda i=i: dec.stream(i) for i in range(K)])
    stream_g.replay()
    sreg = Region(torch, W, stream_g.replay, K, rounds=args.rounds)
    ms_s = sreg.run()
    stream_gbs = dec.wbytes / (ms_s * 1e-3) / 1e9
    traffic = stored_traffic("decode_w4a16_m1", dec.bytes)
    roofline = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": DECODE_KERNEL, "bytes_per_launch": dec.bytes, "us_per_launch": round(ms * 1e3, 3),
                "timing": region.describe(),
                "stream_read_same_footprint": {"bytes": dec.wbytes, "us": round(ms_s * 1e3, 3),
                                               "GB/s": round(stream_gbs, 1), "timing": sreg.describe()},
                "frac_of_stream_read": round(ms_s / ms, 4)}
    del timed_g, warm_g, stream_g
    if args.only == "decode":
        print(json.dumps({"case": "decode", "us_per_launch": roofline["us_per_launch"], "GB/s": roofline["achieved"],
                          "launches_timed": K, "warmup": Wm, "timing": region.describe(),
                          "stream_read_us": roofline["stream_read_same_footprint"]["us"]}), flush=True)
        return

    secondary = {}

    def add_decode(label, M, kind):
        d = Decode(torch, W, M, kind)
        g = graph_of(torch, [lambda i=i: d.launch(i) for i in range(50)])
        g.replay()
        t = Region(torch, W, g.replay, 50, rounds=3).run()
        secondary[label] = {"GB/s": round(d.bytes / (t * 1e-3) / 1e9, 1), "us": round(t * 1e3, 3),
                            "frac_hbm": round(d.bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": d.bytes}
        del g, d

    add_decode("decode_w4a16_m4", 4, "int4")
    add_decode("decode_w4a16_m16", 16, "int4")
    add_decode("decode_w8a16_m1", 1, "e4m3")
    add_decode("decode_w4a16_asym_m1", 1, "int4_asym")
    add_decode("decode_nvfp4_m1", 1, "nvfp4")
    add_decode("decode_nvfp4_m16", 16, "nvfp4")
    torch.cuda.empty_cache()

    pf = Prefill(torch, W)
    with clocks:
        t = time_eager(torch, pf.launch, 10)
    clock_summary["prefill_mxfp4_timed_rounds"] = clocks.summary()
    tf = pf.flops / (t * 1e-3) / 1e12
    secondary["prefill_mxfp4_m8192"] = {"TFLOP/s": round(tf, 1), "frac_bf16_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
                                        "ms": round(t, 3), "flops": pf.flops}
    # secondary denominator: torch.matmul bf16 (hipBLASLt) at the same shape
    # on the same values (the dequantized MXFP4 weights), timed in rounds
    # interleaved with the kernel's
    wb = W.wq_dequant(pf.codes, W.WQ_E2M1X2, pf.sc, W.WQ_E8M0, 32, pf.N, pf.K)
    tk, tt = [], []
    for _ in range(3):
        tk.append(time_eager(torch, pf.launch, 10, warm=1, rounds=1))
        tt.append(time_eager(torch, lambda i: torch.matmul(pf.x, wb.t()), 10, warm=1, rounds=1))
    t2 = float(np.median(tt))
    secondary["torch_matmul_bf16_8192x14336x4096"] = {"TFLOP/s": round(pf.flops / (t2 * 1e-3) / 1e12, 1),
                                                      "ms": round(t2, 3), "weights": "the dequantized MXFP4 weights"}
    secondary["prefill_mxfp4_vs_torch_interleaved"] = {"kernel_ms": [round(v, 3) for v in tk],
                                                      "torch_ms": [round(v, 3) for v in tt],
                                                      "ratio_of_medians": round(float(np.median(tk)) / t2, 4)}
    del pf, wb
    pf = Prefill(torch, W, kind="nvfp4")
    t = time_eager(torch, pf.launch, 10)
    tf = pf.flops / (t * 1e-3) / 1e12
    secondary["prefill_nvfp4_m8192"] = {"TFLOP/s": round(tf, 1), "frac_bf16_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
                                        "ms": round(t, 3)}
    del pf
    torch.cuda.empty_cache()
    for mode in ("block", "channel"):
        g8 = W8A8(torch, W, mode)
        t = time_eager(torch, g8.launch, 10)
        tf = g8.flops / (t * 1e-3) / 1e12
        secondary[f"w8a8_{mode}_8192x14336x4096"] = {"TFLOP/s": round(tf, 1), "frac_fp8_mfma": round(tf / FP8_PEAK_TFLOPS, 4),
                                                     "ms": round(t, 3)}
        del g8
        torch.cuda.empty_cache()

    for kind, rule in (("e4m3", None), ("mxfp4", None), ("mxfp8", "round"), ("mxfp8", "ceil_div")):
        q = ActQuant(torch, W, kind, rule)
        g = graph_of(torch, [lambda i=i: q.launch(i) for i in range(40)])
        g.replay()
        t = time_graph(torch, g, 40)
        label = f"act_quant_{kind}_4096x7168" + (f"_{rule}" if rule else "")
        secondary[label] = {"GB/s": round(q.bytes / (t * 1e-3) / 1e9, 1), "us": round(t * 1e3, 2),
                            "frac_hbm": round(q.bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if kind == "mxfp8" and rule == "round":
            shares = {}
            for elem, block in (("e2m1", 16), ("e2m1", 32), ("e4m3", 32)):
                for r in W.MX_RULES:
                    shares[f"{elem}_b{block}_{r}"] = clip_share(torch, W, q.xs[0], block, elem, r)
            secondary["mx_rule_clip_share_4096x7168"] = shares
        del g, q
    wq_ = WeightQuant(torch, W)
    t = time_eager(torch, wq_.launch, 10)
    secondary["weight_quant_mxfp4_14336x4096_fp32"] = {"GB/s": round(wq_.bytes / (t * 1e-3) / 1e9, 1),
                                                       "us": round(t * 1e3, 2)}
    del wq_
    for which in ("gate_up", "down"):
        mo = MoeW4A8(torch, W, which)
        t = time_eager(torch, mo.launch, 10)
        tf = mo.flops / (t * 1e-3) / 1e12
        secondary[f"moe_w4a8_{which}_64x{mo.N}x{mo.K}_top8"] = {
            "TFLOP/s": round(tf, 1), "frac_fp8_mfma": round(tf / FP8_PEAK_TFLOPS, 4), "us": round(t * 1e3, 1),
            "flops": mo.flops}
        if which == "gate_up":
            t = time_eager(torch, lambda i: W.wq_moe_route(mo.logits, mo.k), 20)
            secondary["moe_route_4096x64_top8"] = {"us": round(t * 1e3, 2)}
            t = time_eager(torch, lambda i: W.quantize_e4m3(mo.x, -1), 20)
            secondary["moe_token_quant_e4m3_4096x4096"] = {"us": round(t * 1e3, 2)}
        t = time_eager(torch, lambda i: W.wq_w4a8_prepack(mo.packed, mo.sb, wq_out=mo.wq), 5)
        secondary[f"moe_w4a8_prepack_{which}"] = {"us": round(t * 1e3, 1)}
        del mo
        torch.cuda.empty_cache()
    cp = Copy(torch)
    t = time_eager(torch, cp.launch, 20)
    secondary["stream_copy_256MiB"] = {"GB/s": round(cp.bytes / (t * 1e-3) / 1e9, 1)}
    del cp
    bs = BigStream(torch, W)
    t = time_eager(torch, bs.launch, 10)
    secondary["stream_read_2GiB"] = {"GB/s": round(bs.bytes / (t * 1e-3) / 1e9, 1), "us": round(t * 1e3, 1)}
    del bs
    torch.cuda.empty_cache()

    cpu = None if args.no_cpu else cpu_baseline()

    line = {
        "metric": "wq_gemm decode GB/s (% HBM peak) at M=1; prefill TFLOP/s (% bf16 MFMA peak)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode W4A16 GEMV: M=1, K=4096, N=14336, INT4 (8 per uint32) with bf16 scales "
                               "per 128-element group; bf16 x with 0.5% channels x30; weights cycled over "
                               f"{len(dec.copies)} resident copies", "parallelism": "none (1 GPU)"},
        "roofline": roofline, "cpu_baseline": cpu, "secondary": secondary,
        "gpu_clocks_hwmon": clock_summary,
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

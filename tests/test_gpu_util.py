"""The measurement utilities on the GPU: the streaming read, the busy kernel
and the clock probe run, end, and report plausible values."""
import pytest
import torch

from tests.gpu_helpers import banner

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    import weight_only_quantized_quant_amd as W
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return W


def test_stream_read_and_spin_complete(W):
    banner("util stream_read 1 MiB + 16 B tail, spin 1000")
    buf = torch.zeros(((1 << 20) + 16) // 4, dtype=torch.int32, device="cuda")
    W.wq_util_stream_read(buf)
    W.wq_util_stream_read(buf, 16)
    W.wq_util_spin(1000)
    torch.cuda.synchronize()


def test_clock_probe_reports_a_plausible_shader_clock(W):
    banner("util clock probe 200 ticks")
    khz = W.wq_util_wall_clock_khz()
    assert 1_000 <= khz <= 1_000_000
    out = torch.zeros(4, dtype=torch.int64, device="cuda")
    W.wq_util_spin(20000)                    # some load first, so the clock is not parked
    W.wq_util_clock(out[:2], 200)
    W.wq_util_clock(out[2:], 1)
    c = out.cpu().tolist()
    assert c[1] >= 200 and c[0] > 0 and c[3] >= 1
    mhz = c[0] / c[1] * khz * 1e-3
    print(f"[clock probe] wall clock {khz} kHz, shader clock {mhz:.0f} MHz over {c[1]} ticks")
    assert 50 <= mhz <= 5000

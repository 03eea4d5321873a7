"""The shader-clock probe (measurement support) returns a plausible clock:
the wait spans at least the requested real-time ticks and the cycle count
corresponds to a clock between 100 MHz and 3 GHz."""
import pytest
import torch

from tests.parity import say

pytestmark = pytest.mark.gpu


def test_clock_probe_alone(fp8q):
    out = torch.zeros(3, dtype=torch.int64, device="cuda")
    ticks = 1_000_000  # 10 ms at 100 MHz
    assert fp8q.fp8q_clock_probe(out.data_ptr(), ticks, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    t, cyc, khz = (int(v) for v in out.cpu())
    khz = khz or 100000
    mhz = cyc / (t / (khz * 1e3)) / 1e6
    say(f"probe: {t} ticks at {khz} kHz, {cyc} cycles -> {mhz:.0f} MHz")
    assert t >= ticks
    assert 100 <= mhz <= 3000

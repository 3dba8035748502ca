"""The shader-clock probe the bench uses to price the matrix cores at the clock they run."""

import pytest

pytestmark = pytest.mark.gpu


def test_clock_probe_reports_a_plausible_clock():
    import torch
    import w4a4_post_quantization_amd as kq
    kq.load()
    out = kq.clock_probe(200)
    torch.cuda.synchronize()
    cycles, ticks = (int(v) for v in out.tolist())
    assert ticks >= 200 * 100                       # at least the requested span of 100 MHz ticks
    mhz = 100.0 * cycles / ticks
    print(f"idle shader clock {mhz:.0f} MHz")
    assert 50.0 < mhz < 3000.0

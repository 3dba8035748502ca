"""The measurement helpers the bench uses: the shader-clock probe (the matrix cores priced at
the clock they run) and the FP4 matrix-core rate probe."""

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


def test_mfma_fp4_probe_sums():
    """Each wavefront's sum equals its products' total: with every lane holding the same
    operands, one 32x32x64 product is 2 * (the 32 codes' dot product) per output, and each
    round adds four each of A.B, B.A, A.A and B.B over 1024 outputs."""
    import numpy as np
    import torch
    import w4a4_post_quantization_amd as kq
    kq.load()
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
    rng = np.random.default_rng(7)
    a = rng.integers(0, 256, 16, dtype=np.uint8)            # one lane's 16 bytes, the same in every lane
    b = rng.integers(0, 256, 16, dtype=np.uint8)
    codes = np.concatenate([np.tile(a, 64), np.tile(b, 64)])
    dev = torch.from_numpy(codes).cuda()
    iters, wgs = 50, 8
    out = kq.mfma_fp4_probe(iters, wgs, dev)
    torch.cuda.synchronize()
    def vals(byts):                                          # 32 codes, low nibble first
        return np.array([e2m1[(int(x) >> s) & 15] for x in byts for s in (0, 4)])
    va, vb = vals(a), vals(b)
    # a lane pair (l, l + 32) holds k-blocks 0 and 1 of the 64-wide product, each 32 codes
    dot = lambda x, y: 2.0 * float(np.dot(x, y))
    per_output = 4 * (dot(va, vb) * 2 + dot(va, va) + dot(vb, vb))
    expect = iters * per_output * 32 * 32
    got = out.cpu().numpy()
    assert got.shape == (4 * wgs,)
    assert np.allclose(got, expect, rtol=1e-5, atol=1e-3), (got[:4], expect)

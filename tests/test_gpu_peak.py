"""The matrix-core loop yardstick (moe_mfma_loop) on the device: it runs, its
FLOP count is the launch's, and the clock it reports is a plausible shader
clock. Not a parity test: the loop computes nothing the layer uses."""
import math

import pytest
import torch

import mixture_experts_layer_10_amd as moe

pytestmark = pytest.mark.gpu


def test_mfma_loop_runs_and_reports_clock():
    out = torch.zeros(3, dtype=torch.int64, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    flops = moe.mfma_loop(iters, out)
    torch.cuda.synchronize()
    # 2 workgroups x 4 wavefronts per CU, 4 MFMAs of 2*32*32*16 FLOPs per iteration
    assert flops == 2 * cus * 4 * iters * 4 * 2 * 32 * 32 * 16
    ticks, rt, chk = out.tolist()
    assert ticks > 0 and rt > 0
    mhz = ticks / rt * 100.0
    print(f"mfma loop: {cus} CUs, shader clock {mhz:.0f} MHz over {rt / 100:.0f} us")
    assert 300.0 < mhz < 3000.0
    s = torch.tensor([chk], dtype=torch.int64).to(torch.int32).view(torch.float32).item()
    assert math.isfinite(s)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16 * 7, 3 * (1 << 20) + 16 * 33])
def test_stream_read_reads_every_granule(nbytes):
    """The fold covers every 16-byte granule, ragged tails included: a buffer
    whose only nonzero word is the marker (at the start, the middle or the
    last granule) folds to the marker, which the kernel then stores."""
    n = nbytes // 4
    for pos in (0, n // 2, n - 1):
        buf = torch.zeros(n, dtype=torch.int32, device="cuda")
        buf[pos] = torch.tensor(0x9E3779B9, dtype=torch.int64).to(torch.int32)
        out = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        assert moe.stream_read(buf, out) == nbytes
        torch.cuda.synchronize()
        assert out.item() == torch.tensor(0x9E3779B9, dtype=torch.int64).to(torch.int32).item(), (nbytes, pos)
    buf = torch.zeros(n, dtype=torch.int32, device="cuda")
    out = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    moe.stream_read(buf, out)
    torch.cuda.synchronize()
    assert out.item() == 7                       # fold 0: nothing written

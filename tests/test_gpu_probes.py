"""The measurement probes of include/qmm_probe.h on the GPU: the read probe
leaves its sink untouched (the data it reads never equals the magic word),
the empty kernel runs, and the clock probe's readings are monotone and give
a shader clock in a plausible range for every workgroup."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
from skinny_bit_block_amd import probe  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_read_and_empty_probes():
    buf = torch.full((64 << 20,), 3, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for grid, block in ((1, 64), (7, 256), (1024, 512)):
        probe.qmm_probe_read(buf.data_ptr(), buf.numel(), grid, block, sink.data_ptr(), stream())
    probe.qmm_probe_read(buf.data_ptr(), 16, 3, 64, sink.data_ptr(), stream())  # fewer units than workgroups
    probe.qmm_probe_empty(256, stream())
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("grid", [1, 256, 1024])
def test_clock_probe(grid):
    counts = torch.full((4 * grid + 4,), -1, dtype=torch.int64, device="cuda")
    khz = probe.qmm_probe_clock(counts.data_ptr(), grid, 1 << 16, stream())
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert c[-4:].tolist() == [-1] * 4  # nothing past 4 * grid words
    c = c[:-4].reshape(grid, 4).astype(np.float64)
    assert khz > 0
    assert (c[:, 2] > c[:, 0]).all() and (c[:, 3] > c[:, 1]).all()
    ghz = (c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]) * khz * 1e-6
    assert ((ghz > 0.3) & (ghz < 5.0)).all(), (ghz.min(), ghz.max())

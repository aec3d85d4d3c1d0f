"""GPU parity of the block-scaled FP4 product (qmm_run_nvfp4, through the C
ABI) against the binary64 oracle (oracle/nvfp4.py).

Gate per element: |y_gpu - y| <= 2e-3 * sum_k |w[n,k] x[m,k]| (the product's
tolerance; the weights are exact in the kernel, only the binary16 rounding of
x and fp32 accumulation remain), bitwise repeatability, signed and zero scale
codes, forced launch shapes, sampled rows at full size and the argument checks
on a device. Inputs: seeded synthetic codes (synth.nvfp4) and N(0,1) x.
"""
import numpy as np
import pytest

import synth
from oracle import nvfp4 as fp4

torch = pytest.importorskip("torch")
import skinny_bit_block_amd as sbb  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 2e-3
SEED = 20261202


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    handle = sbb.qmm_create(0)
    yield handle
    sbb.qmm_destroy(handle)


def run(h, x, groups, tscale, N, K, shape=(0, 0, 0), wave_splits=0, fill=np.nan):
    M = x.shape[0]
    sbb.qmm_set_shape(h, *shape)
    sbb.qmm_set_wave_splits(h, wave_splits)
    try:
        xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        gd = torch.from_numpy(np.ascontiguousarray(groups).reshape(-1)).cuda()
        y = torch.full((M, N), fill, dtype=torch.float32, device="cuda")
        sbb.qmm_run_nvfp4(h, xd, gd, tscale, y, M, N, K)
        torch.cuda.synchronize()
        return y.cpu().numpy()
    finally:
        sbb.qmm_set_shape(h, 0, 0, 0)
        sbb.qmm_set_wave_splits(h, 0)


def check(y, yref, aref, what=""):
    assert np.all(np.isfinite(y)), what
    err = np.abs(y.astype(np.float64) - yref)
    bad = err > TOL * aref
    assert not bad.any(), "%s: %d of %d outside the gate, worst err/A %.3g" % (
        what, int(bad.sum()), bad.size, float((err / np.maximum(aref, 1e-300)).max()))


def case(M, N, K, tensor, tscale=0.37):
    elems, scales = synth.nvfp4(N, K, tensor=tensor, seed=SEED)
    x = synth.acts(M, K, tensor=tensor + 1, seed=SEED)
    groups = sbb.qmm_nvfp4_repack(elems, scales, N, K)
    yref, aref = fp4.qmm_nvfp4(x, elems, scales, tscale, N, K)
    return x, elems, scales, groups, yref, aref


@pytest.mark.parametrize("M,N,K", [(1, 300, 1280), (2, 64, 256), (4, 300, 2560), (7, 1000, 1280),
                                   (8, 17, 512), (9, 300, 768), (16, 300, 1280), (17, 100, 512),
                                   (32, 300, 1280), (3, 5000, 256)])
def test_parity(h, M, N, K):
    x, _, _, groups, yref, aref = case(M, N, K, tensor=100 + M)
    check(run(h, x, groups, 0.37, N, K), yref, aref, "M=%d N=%d K=%d" % (M, N, K))


# K far beyond the workloads' (thousands of K slices over few row tiles); the
# host address replay walks the same plans
@pytest.mark.parametrize("M,N,K", [(1, 1, 1 << 22), (7, 5, 1 << 20), (32, 3, 1 << 18)])
def test_long_k(h, M, N, K):
    x, _, _, groups, yref, aref = case(M, N, K, tensor=700 + M)
    check(run(h, x, groups, 0.37, N, K), yref, aref, "long K: M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("shape,wsplit", [((4, 1, 0), 1), ((8, 2, 0), 1), ((4, 5, 1), 1),
                                          ((4, 2, 0), 2), ((8, 10, 3), 2), ((2, 3, 1), 1)])
@pytest.mark.parametrize("M", [1, 7, 16])
def test_launch_shapes(h, M, shape, wsplit):
    N, K = 600, 2560
    x, _, _, groups, yref, aref = case(M, N, K, tensor=200 + M, tscale=1.0)
    check(run(h, x, groups, 1.0, N, K, shape=shape, wave_splits=wsplit), yref, aref,
          "M=%d shape=%s wsplit=%d" % (M, shape, wsplit))


def test_signed_and_zero_scales(h):
    M, N, K = 4, 48, 512
    elems, scales = synth.nvfp4(N, K, tensor=301, seed=SEED)
    scales = scales.copy()
    scales[::3] |= 0x80          # negative scale codes
    scales[1::5, ::2] = 0x00     # zero scales
    scales[2::7, 1::3] = 0x03    # subnormal scales
    x = synth.acts(M, K, tensor=302, seed=SEED)
    groups = sbb.qmm_nvfp4_repack(elems, scales, N, K)
    yref, aref = fp4.qmm_nvfp4(x, elems, scales, -2.5, N, K)
    check(run(h, x, groups, -2.5, N, K), yref, aref, "signed/zero scales")


def test_one_hot_weight(h):
    # one nonzero weight: y picks x at that column times its value
    M, N, K = 3, 16, 512
    elems = np.zeros((N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 16), 0x38, dtype=np.uint8)  # 1.0
    n0, k0 = 5, 301
    elems[n0, k0 // 2] = 0x7 << (4 * (k0 % 2))  # 6.0
    scales[n0, k0 // 16] = 0x40  # 2.0
    x = synth.acts(M, K, tensor=303, seed=SEED)
    groups = sbb.qmm_nvfp4_repack(elems, scales, N, K)
    y = run(h, x, groups, 0.5, N, K)
    want = np.zeros((M, N))
    want[:, n0] = 0.5 * 2.0 * 6.0 * x[:, k0].astype(np.float16).astype(np.float64)
    assert np.array_equal(y.astype(np.float64), want)


def test_repeat_is_bitwise_identical(h):
    M, N, K = 7, 700, 2560
    x, _, _, groups, _, _ = case(M, N, K, tensor=400)
    a = run(h, x, groups, 0.37, N, K)
    b = run(h, x, groups, 0.37, N, K)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("M", [1, 4, 7, 16])
def test_full_size_sampled_rows(h, M):
    # gate+up shape, the pages' FP4 bench shape with the most rows per call
    N, K = 34816, 5120
    elems, scales = synth.nvfp4(N, K, tensor=500, seed=SEED)
    x = synth.acts(M, K, tensor=501, seed=SEED)
    groups = sbb.qmm_nvfp4_repack(elems, scales, N, K)
    y = run(h, x, groups, 0.37, N, K)
    rows = np.r_[0:5, 16:21, N // 2 - 3:N // 2 + 3, N - 7:N]
    yref, aref = fp4.qmm_nvfp4(x, elems, scales, 0.37, N, K, rows=rows)
    check(y[:, rows], yref, aref, "full size M=%d" % M)
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("M", [1, 7])
def test_lm_head_bench_shape_sampled_rows(h, M):
    # the 248,320-row lm_head the FP4 bench times (the pages' FP4 bench shape)
    N, K = 248320, 5120
    elems, scales = synth.nvfp4(N, K, tensor=510, seed=SEED)
    x = synth.acts(M, K, tensor=511, seed=SEED)
    groups = sbb.qmm_nvfp4_repack(elems, scales, N, K)
    y = run(h, x, groups, 0.5, N, K)
    rows = np.r_[0:4, 9999:10003, N // 2:N // 2 + 4, N - 4:N]
    yref, aref = fp4.qmm_nvfp4(x, elems, scales, 0.5, N, K, rows=rows)
    check(y[:, rows], yref, aref, "lm_head M=%d" % M)
    assert np.all(np.isfinite(y))


def test_errors_launch_nothing(h):
    M, N, K = 2, 32, 256
    x = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    g = torch.zeros(sbb.qmm_weight_bytes(N, K), dtype=torch.uint8, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    st = sbb._stream(None)
    assert sbb.qmm_run_nvfp4_raw(h, x.data_ptr(), g.data_ptr(), float("nan"), y.data_ptr(), M, N,
                                 K, st) == sbb.QMM_ERR_INVALID_ARG
    assert sbb.qmm_run_nvfp4_raw(h, x.data_ptr(), g.data_ptr(), 1.0, y.data_ptr(), M, N, 300,
                                 st) == sbb.QMM_ERR_SHAPE
    assert sbb.qmm_run_nvfp4_raw(h, x.data_ptr(), g.data_ptr(), 1.0, x.data_ptr(), M, N, K,
                                 st) == sbb.QMM_ERR_OVERLAP
    sbb.qmm_set_kernel(h, sbb.KERNEL_VECTOR)
    try:
        assert sbb.qmm_run_nvfp4_raw(h, x.data_ptr(), g.data_ptr(), 1.0, y.data_ptr(), M, N, K,
                                     st) == sbb.QMM_ERR_INVALID_ARG
    finally:
        sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)

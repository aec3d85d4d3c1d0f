"""GPU parity of the plain INT4 product (qmm_run_int4, through the C ABI)
against the binary64 oracle (oracle/int4.py).

Gate per element: |y_gpu - y| <= 2e-3 * sum_k |w[n,k] x[m,k]| (the product's
tolerance; the codes are exact in the kernel and the scales are applied in
fp32, so only the binary16 rounding of x and fp32 accumulation remain),
exact zeros for zero codes, bitwise repeatability, negative, zero and
subnormal scales, forced launch shapes, sampled rows at full size and the
argument checks on a device. Inputs: seeded synthetic codes and scales
(synth.int4) and N(0,1) x.
"""
import numpy as np
import pytest

import synth
from oracle import int4

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


def run(h, x, groups, N, K, shape=(0, 0, 0), wave_splits=0, fill=np.nan):
    M = x.shape[0]
    sbb.qmm_set_shape(h, *shape)
    sbb.qmm_set_wave_splits(h, wave_splits)
    try:
        xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        gd = torch.from_numpy(np.ascontiguousarray(groups).reshape(-1)).cuda()
        y = torch.full((M, N), fill, dtype=torch.float32, device="cuda")
        sbb.qmm_run_int4(h, xd, gd, y, M, N, K)
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


def case(M, N, K, tensor):
    codes, scales = synth.int4(N, K, tensor=tensor, seed=SEED)
    x = synth.acts(M, K, tensor=tensor + 1, seed=SEED)
    groups = sbb.qmm_int4_repack(codes, scales, N, K)
    yref, aref = int4.qmm_int4(x, codes, scales, N, K)
    return x, codes, scales, groups, yref, aref


# several row tiles and a ragged last tile, K of 1..10 groups, 1..32 rows
@pytest.mark.parametrize("M,N,K", [(1, 300, 1280), (2, 64, 256), (4, 300, 2560), (7, 1000, 1280),
                                   (8, 33, 512), (9, 200, 768), (16, 129, 2560), (17, 64, 1024),
                                   (32, 250, 1536), (3, 1, 256)])
def test_parity(h, M, N, K):
    x, _, _, groups, yref, aref = case(M, N, K, tensor=100 + M + N)
    check(run(h, x, groups, N, K), yref, aref, "M=%d N=%d K=%d" % (M, N, K))


# K far beyond the workloads' (thousands of K slices over few row tiles); the
# host address replay walks the same plans
@pytest.mark.parametrize("M,N,K", [(1, 1, 1 << 22), (7, 5, 1 << 20), (32, 3, 1 << 18)])
def test_long_k(h, M, N, K):
    x, _, _, groups, yref, aref = case(M, N, K, tensor=700 + M)
    check(run(h, x, groups, N, K), yref, aref, "long K: M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("shape,wsplit", [((4, 1, 0), 1), ((8, 2, 0), 1), ((4, 5, 1), 1),
                                          ((4, 2, 0), 2), ((8, 10, 3), 2), ((2, 3, 1), 1),
                                          ((6, 2, 0), 2), ((3, 1, 0), 1)])
@pytest.mark.parametrize("M", [1, 7, 16])
def test_launch_shapes(h, M, shape, wsplit):
    N, K = 600, 2560
    x, _, _, groups, yref, aref = case(M, N, K, tensor=200 + M)
    check(run(h, x, groups, N, K, shape=shape, wave_splits=wsplit), yref, aref,
          "M=%d shape=%s wsplit=%d" % (M, shape, wsplit))


def test_negative_zero_and_subnormal_scales(h):
    M, N, K = 4, 48, 512
    codes, scales = synth.int4(N, K, tensor=301, seed=SEED)
    scales = scales.copy()
    scales[::3] |= 0x8000        # negative scales
    scales[1::5, ::2] = 0x0000   # zero scales
    scales[2::7, 1::3] = 0x0011  # subnormal scales
    x = synth.acts(M, K, tensor=302, seed=SEED)
    groups = sbb.qmm_int4_repack(codes, scales, N, K)
    yref, aref = int4.qmm_int4(x, codes, scales, N, K)
    check(run(h, x, groups, N, K), yref, aref, "negative/zero/subnormal scales")


def test_zero_codes_give_exact_zeros(h):
    # q = 0 everywhere (stored as 8): the exact decode leaves nothing behind
    M, N, K = 5, 40, 768
    _, scales = synth.int4(N, K, tensor=305, seed=SEED)
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    x = synth.acts(M, K, tensor=306, seed=SEED)
    groups = sbb.qmm_int4_repack(codes, scales, N, K)
    y = run(h, x, groups, N, K)
    assert np.array_equal(y, np.zeros((M, N), dtype=np.float32))


def test_one_hot_weight(h):
    # one nonzero weight (code -8, the most negative): y picks x at that column
    M, N, K = 3, 16, 512
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 128), 0x3C00, dtype=np.uint16)  # 1.0
    n0, k0 = 5, 301
    codes[n0, k0 // 2] = 0x8 << (4 * (k0 % 2))  # -8
    scales[n0, k0 // 128] = 0x3E00  # 1.5
    x = synth.acts(M, K, tensor=303, seed=SEED)
    groups = sbb.qmm_int4_repack(codes, scales, N, K)
    y = run(h, x, groups, N, K)
    want = np.zeros((M, N))
    want[:, n0] = 1.5 * -8.0 * x[:, k0].astype(np.float16).astype(np.float64)
    assert np.array_equal(y.astype(np.float64), want)


def test_each_scale_group_reaches_its_weights(h):
    # codes 1 everywhere; one row per scale slot with that slot at 2.0: the
    # output moves by exactly the x of that slot's 128 columns
    M, N, K = 2, 8, 1024
    codes = np.full((N, K // 2), 0x11, dtype=np.uint8)
    scales = np.full((N, K // 128), 0x3C00, dtype=np.uint16)
    for n in range(N):
        scales[n, n] = 0x4000
    x = synth.acts(M, K, tensor=307, seed=SEED)
    groups = sbb.qmm_int4_repack(codes, scales, N, K)
    yref, aref = int4.qmm_int4(x, codes, scales, N, K)
    check(run(h, x, groups, N, K), yref, aref, "scale slots")


def test_repeat_is_bitwise_identical(h):
    M, N, K = 7, 700, 2560
    x, _, _, groups, _, _ = case(M, N, K, tensor=400)
    a = run(h, x, groups, N, K)
    b = run(h, x, groups, N, K)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("M", [1, 4, 7, 16])
def test_full_size_sampled_rows(h, M):
    # the gate+up shape at full size
    N, K = 34816, 5120
    codes, scales = synth.int4(N, K, tensor=500, seed=SEED)
    x = synth.acts(M, K, tensor=501, seed=SEED)
    groups = sbb.qmm_int4_repack(codes, scales, N, K)
    y = run(h, x, groups, N, K)
    rows = np.r_[0:5, 16:21, N // 2 - 3:N // 2 + 3, N - 7:N]
    yref, aref = int4.qmm_int4(x, codes, scales, N, K, rows=rows)
    check(y[:, rows], yref, aref, "full size M=%d" % M)
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("shape", ["square", "down", "lm_head"])
@pytest.mark.parametrize("M", [1, 7, 16, 32])
def test_pass_shapes_sampled_rows(h, shape, M):
    # the other matrices of the model pass, in the launch shapes their table
    # entries pick
    N, K = {"square": (5120, 5120), "down": (5120, 17408), "lm_head": (151936, 5120)}[shape]
    codes, scales = synth.int4(N, K, tensor=520 + N % 97, seed=SEED)
    x = synth.acts(M, K, tensor=521, seed=SEED)
    groups = sbb.qmm_int4_repack(codes, scales, N, K)
    y = run(h, x, groups, N, K)
    rows = np.r_[0:4, 1000:1004, N // 2:N // 2 + 4, N - 4:N]
    yref, aref = int4.qmm_int4(x, codes, scales, N, K, rows=rows)
    check(y[:, rows], yref, aref, "%s M=%d" % (shape, M))
    assert np.all(np.isfinite(y))


def test_errors_launch_nothing(h):
    M, N, K = 2, 32, 256
    x = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    g = torch.zeros(sbb.qmm_weight_bytes(N, K), dtype=torch.uint8, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    st = sbb._stream(None)
    assert sbb.qmm_run_int4_raw(h, x.data_ptr(), g.data_ptr(), y.data_ptr(), M, N, 300,
                                st) == sbb.QMM_ERR_SHAPE
    assert sbb.qmm_run_int4_raw(h, x.data_ptr(), g.data_ptr(), x.data_ptr(), M, N, K,
                                st) == sbb.QMM_ERR_OVERLAP
    sbb.qmm_set_kernel(h, sbb.KERNEL_VECTOR)
    try:
        assert sbb.qmm_run_int4_raw(h, x.data_ptr(), g.data_ptr(), y.data_ptr(), M, N, K,
                                    st) == sbb.QMM_ERR_INVALID_ARG
    finally:
        sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)

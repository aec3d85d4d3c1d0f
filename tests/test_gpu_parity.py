"""GPU parity: the HIP path (through the C ABI) against the binary64 oracle.

Gate per element: |y_gpu - y| <= 2e-3 * sum_k |w[n,k] x[m,k]| (the tolerance
of the product, derived in the oracle's and the header's terms), plus exact
bitwise repeatability, one-hot read-outs of the dequantized matrix, binary16
subnormal scales, zero scales and the argument checks of qmm_run on a device.
Inputs are seeded synthetic tensors with the distributions of the workloads
(tests/../synth).
"""
import os

import numpy as np
import pytest

import oracle
import synth
import workload_cases as wc

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


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(h, x, W, N, K, kernel=sbb.KERNEL_AUTO, shape=(0, 0, 0), fill=np.nan, wave_splits=0):
    M = x.shape[0]
    sbb.qmm_set_kernel(h, kernel)
    sbb.qmm_set_shape(h, *shape)
    sbb.qmm_set_wave_splits(h, wave_splits)
    try:
        xd, Wd = to_dev(x), to_dev(W.reshape(-1))
        y = torch.full((M, N), fill, dtype=torch.float32, device="cuda")
        sbb.qmm_run(h, xd, Wd, y, M, N, K)
        torch.cuda.synchronize()
        return y.cpu().numpy()
    finally:
        sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)
        sbb.qmm_set_shape(h, 0, 0, 0)
        sbb.qmm_set_wave_splits(h, 0)


def run_chunked(h, x, W, N, K, kernel):
    # the row-vector kernel takes at most 8 rows per call
    step = 8 if kernel == sbb.KERNEL_VECTOR else x.shape[0]
    return np.concatenate([run(h, x[i:i + step], W, N, K, kernel=kernel)
                           for i in range(0, x.shape[0], step)])


def check(y, yref, aref, what=""):
    err = np.abs(y.astype(np.float64) - yref)
    assert np.all(np.isfinite(y)), what
    bad = err > TOL * aref
    if bad.any():
        m, n = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements outside the gate; first (m=%d, n=%d): gpu %.9g "
                             "oracle %.9g gate %.3g" % (what, bad.sum(), m, n, y[m, n],
                                                        yref[m, n], TOL * aref[m, n]))
    ratio = float((err / np.maximum(aref, 1e-300)).max())
    if ratio > 1e-4:
        print("%s: max err/A = %.3g (above 1e-4)" % (what, ratio))
    return ratio


def inputs(M, N, K, tag, xscale=1.0):
    W = synth.weights(N, K, tensor=1000 + tag, seed=SEED)
    x = synth.acts(M, K, tensor=2000 + tag, seed=SEED, scale=xscale)
    return x, W


def sample_rows(N, count=384, seed=0):
    rng = np.random.default_rng(seed)
    edge = [0, 1, 15, 16, 17, N // 2, N - 17, N - 16, N - 2, N - 1]
    rows = np.unique(np.concatenate([rng.integers(0, N, count), [r for r in edge if 0 <= r < N]]))
    return rows


# ------------------------------------------------------------------ small shapes

SMALL_NK = [(1, 256), (3, 512), (17, 1280), (129, 256), (2047, 512), (40, 2560)]


@pytest.mark.parametrize("N,K", SMALL_NK)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 7, 8])
def test_small_vector(h, M, N, K):
    x, W = inputs(M, N, K, tag=N + K + M)
    y = run(h, x, W, N, K, kernel=sbb.KERNEL_VECTOR)
    yref, aref = oracle.qmm(x, W, N, K)
    check(y, yref, aref, "vector M=%d N=%d K=%d" % (M, N, K))


@pytest.mark.parametrize("N,K", SMALL_NK)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 8, 9, 13, 16, 17, 32])
def test_small_tiled(h, M, N, K):
    x, W = inputs(M, N, K, tag=N + K + M + 7)
    y = run(h, x, W, N, K, kernel=sbb.KERNEL_TILED)
    yref, aref = oracle.qmm(x, W, N, K)
    check(y, yref, aref, "tiled M=%d N=%d K=%d" % (M, N, K))


# K far beyond the workloads', up to the largest the library takes (2^24):
# thousands of K slices over one to three row tiles (the same cases the host
# address replay walks)
LONG_K = [(1, 1 << 24, 1, sbb.KERNEL_AUTO), (1, 1 << 24, 1, sbb.KERNEL_TILED),
          (1, 1 << 24, 7, sbb.KERNEL_AUTO), (1, 1 << 24, 7, sbb.KERNEL_VECTOR),
          (17, 1 << 22, 1, sbb.KERNEL_AUTO), (17, 1 << 22, 7, sbb.KERNEL_VECTOR),
          (20, 1 << 20, 7, sbb.KERNEL_AUTO), (20, 1 << 20, 32, sbb.KERNEL_AUTO),
          (5, 1 << 19, 32, sbb.KERNEL_AUTO), (33, 1 << 18, 1, sbb.KERNEL_TILED),
          (33, 1 << 18, 32, sbb.KERNEL_AUTO)]


@pytest.mark.parametrize("N,K,M,kernel", LONG_K)
def test_long_k(h, N, K, M, kernel):
    x, W = inputs(M, N, K, tag=N + M + kernel + (K >> 18))
    y = run(h, x, W, N, K, kernel=kernel)
    yref, aref = oracle.qmm(x, W, N, K)
    check(y, yref, aref, "long K: M=%d N=%d K=%d kernel %d" % (M, N, K, kernel))


@pytest.mark.parametrize("shape", [(1, 1, 0), (2, 3, 0), (4, 2, 0), (8, 5, 0), (8, 1, 0), (1, 10, 0),
                                   (4, 7, 500), (8, 4, 63),
                                   # fewer workgroups than tiles: waves walk several tiles
                                   (1, 1, 1), (2, 3, 5), (4, 1, 3), (8, 2, 1), (4, 10, 2)])
@pytest.mark.parametrize("M,kernel", [(5, sbb.KERNEL_VECTOR), (12, sbb.KERNEL_TILED),
                                      (8, sbb.KERNEL_VECTOR), (3, sbb.KERNEL_TILED)])
def test_launch_shapes(h, M, kernel, shape):
    N, K = 1000, 2560
    x, W = inputs(M, N, K, tag=31 + M)
    y = run(h, x, W, N, K, kernel=kernel, shape=shape)
    yref, aref = oracle.qmm(x, W, N, K)
    check(y, yref, aref, "M=%d kernel=%d shape=%s" % (M, kernel, shape))


# K slices reduced inside a workgroup (in LDS), alone and combined with split-K
# across workgroups, with persistent grids and with waves whose slice lies past
# the end of K (10 super-blocks here)
@pytest.mark.parametrize("shape,wsplit", [((2, 2, 0), 2), ((4, 4, 0), 4), ((5, 5, 0), 5),
                                          ((4, 8, 0), 4), ((8, 4, 0), 4), ((6, 3, 0), 3),
                                          ((8, 8, 3), 2), ((4, 10, 1), 2), ((3, 3, 2), 3),
                                          ((8, 10, 0), 8), ((7, 7, 0), 7),
                                          ((2, 10, 0), 2), ((4, 10, 0), 4)])
@pytest.mark.parametrize("M,kernel", [(1, sbb.KERNEL_VECTOR), (5, sbb.KERNEL_VECTOR),
                                      (3, sbb.KERNEL_TILED), (12, sbb.KERNEL_TILED),
                                      (20, sbb.KERNEL_TILED)])
def test_wave_splits(h, M, kernel, shape, wsplit):
    N, K = 1000, 2560
    sbb.qmm_set_kernel(h, kernel)
    sbb.qmm_set_shape(h, *shape)
    sbb.qmm_set_wave_splits(h, wsplit)
    try:
        sbb.qmm_query_plan(h, M, N, K)
    except sbb.QmmError as e:
        assert e.status == sbb.QMM_ERR_INVALID_ARG
        pytest.skip("this launch shape does not fit the LDS at M=%d" % M)
    finally:
        sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)
        sbb.qmm_set_shape(h, 0, 0, 0)
        sbb.qmm_set_wave_splits(h, 0)
    x, W = inputs(M, N, K, tag=47 + M)
    y = run(h, x, W, N, K, kernel=kernel, shape=shape, wave_splits=wsplit)
    yref, aref = oracle.qmm(x, W, N, K)
    check(y, yref, aref, "M=%d kernel=%d shape=%s wave_splits=%d" % (M, kernel, shape, wsplit))


# ------------------------------------------------------------ the workloads

WORKLOAD_PARAMS = wc.params()


@pytest.mark.parametrize("name,N,K,M,xscale", WORKLOAD_PARAMS)
def test_workload_shape(h, name, N, K, M, xscale):
    # the whole output of one call at the library's own plan (the plan the
    # benchmark times) against the oracle; y starts NaN-filled, so an
    # unwritten tile fails the finiteness check
    tag = {"single_2048": 0, "gate_up": 1, "down": 2, "lm_head": 3, "square_5120": 4,
           "fused_5x5120": 5}[name]
    x, W = inputs(M, N, K, tag=tag, xscale=xscale)
    y = run(h, x, W, N, K)
    yref, aref = oracle.qmm(x, W, N, K)
    check(y, yref, aref, "%s M=%d" % (name, M))


# ---------------------------------------------------- probes and special cases

@pytest.mark.parametrize("kernel", [sbb.KERNEL_VECTOR, sbb.KERNEL_TILED])
def test_one_hot_reads_out_the_matrix(h, kernel):
    # x = e_k: y[m, n] = w[n, k_m]. Checked against the oracle's dequantized
    # weights at 2e-3 * |w|, tighter than the row gate.
    N, K, M = 333, 1536, 32
    W = synth.weights(N, K, tensor=77, seed=SEED)
    ks = np.array([0, 1, 2, 3, 4, 31, 32, 33, 63, 64, 95, 96, 127, 128, 191, 192, 255,
                   256, 300, 511, 512, 700, 767, 768, 1000, 1023, 1024, 1100, 1279, 1280,
                   1400, 1535])
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y = run_chunked(h, x, W, N, K, kernel)
    w = oracle.dequant_rows(W, N, K, np.arange(N))
    ref = w[:, ks].T
    assert np.all(np.abs(y - ref) <= TOL * np.abs(ref)), np.abs(y - ref).max()


@pytest.mark.parametrize("kernel", [sbb.KERNEL_VECTOR, sbb.KERNEL_TILED])
def test_subnormal_scales(h, kernel):
    # every d and dmin a binary16 subnormal: a flush to zero would give y = 0
    # or drop the min term; the row gate alone does not see that, the one-hot
    # read-out does.
    N, K, M = 200, 1024, 16
    rng = np.random.default_rng(5)
    Wb = synth.weights(N, K, tensor=78, seed=SEED).reshape(N, K // 256, 144).copy()
    d = rng.integers(1, 1024, size=(N, K // 256)).astype(np.uint16)
    dm = rng.integers(1, 1024, size=(N, K // 256)).astype(np.uint16)
    Wb[:, :, 0] = d & 0xFF
    Wb[:, :, 1] = d >> 8
    Wb[:, :, 2] = dm & 0xFF
    Wb[:, :, 3] = dm >> 8
    W = Wb.reshape(N, -1)
    x, _ = inputs(M, N, K, tag=79)
    y = run_chunked(h, x, W, N, K, kernel)
    yref, aref = oracle.qmm(x, W, N, K)
    check(y, yref, aref, "subnormal d/dmin")
    ks = np.arange(0, K, K // M)[:M] + 5
    xo = np.zeros((M, K), dtype=np.float32)
    xo[np.arange(M), ks] = 1.0
    yo = run_chunked(h, xo, W, N, K, kernel)
    ref = oracle.dequant_rows(W, N, K, np.arange(N))[:, ks].T
    assert np.mean(ref != 0) > 0.9  # a few weights are exactly 0 (q = 0 with m = 0)
    assert np.all(np.abs(yo - ref) <= TOL * np.abs(ref))


@pytest.mark.parametrize("kernel", [sbb.KERNEL_VECTOR, sbb.KERNEL_TILED])
def test_zero_scales_give_zero(h, kernel):
    N, K, M = 100, 768, 8
    x, W = inputs(M, N, K, tag=80)
    Wb = W.reshape(N, K // 256, 144).copy()
    Wb[:, :, 0:4] = 0
    y = run(h, x, Wb.reshape(N, -1), N, K, kernel=kernel)
    assert np.all(y == 0.0)
    Wb = W.reshape(N, K // 256, 144).copy()
    Wb[:, :, 4:16] = 0
    y = run(h, x, Wb.reshape(N, -1), N, K, kernel=kernel)
    assert np.all(y == 0.0)


def test_largest_scales(h):
    # d = 65504, sc = 63, q = 15 everywhere, dmin = 0: w = 61901280
    N, K, M = 48, 512, 8
    Wb = np.zeros((N, K // 256, 144), dtype=np.uint8)
    Wb[:, :, 0:2] = [0xFF, 0x7B]
    Wb[:, :, 4:8] = 0xFF
    Wb[:, :, 12:16] = 0x0F
    Wb[:, :, 16:] = 0xFF
    W = Wb.reshape(N, -1)
    x, _ = inputs(M, N, K, tag=81)
    yref, aref = oracle.qmm(x, W, N, K)
    for kernel in (sbb.KERNEL_VECTOR, sbb.KERNEL_TILED):
        check(run(h, x, W, N, K, kernel=kernel), yref, aref, "largest d")


def test_rows_match_single_row_passes(h):
    # row i of an M-row pass and the M = 1 pass of that row agree within the gate
    N, K, M = 4096, 5120, 16
    x, W = inputs(M, N, K, tag=82)
    yM = run(h, x, W, N, K)
    rows = sample_rows(N, 64)
    yref, aref = oracle.qmm_rows(x, W, N, K, rows)
    for m in range(M):
        y1 = run(h, x[m:m + 1], W, N, K)
        assert np.all(np.abs(yM[m] - y1[0]).astype(np.float64)[rows] <= TOL * aref[m])


# -------------------------------------------------------------- determinism

@pytest.mark.parametrize("M,N,K,kernel", [
    (4, 2048, 2048, 0), (1, 34816, 5120, 0), (8, 34816, 5120, 0), (16, 34816, 5120, 0),
    (4, 5120, 17408, 0), (16, 5120, 17408, 0), (7, 151936, 5120, 0), (32, 5120, 5120, 0),
    (7, 5120, 5120, sbb.KERNEL_VECTOR)])
def test_bitwise_repeatable(h, M, N, K, kernel):
    x, W = inputs(M, N, K, tag=90 + M)
    sbb.qmm_set_kernel(h, kernel)
    try:
        xd, Wd = to_dev(x), to_dev(W.reshape(-1))
        outs = []
        for _ in range(5):
            y = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
            sbb.qmm_run(h, xd, Wd, y, M, N, K)
            outs.append(y)
        torch.cuda.synchronize()
        ref = outs[0].cpu().numpy().view(np.uint32)
        for o in outs[1:]:
            assert np.array_equal(o.cpu().numpy().view(np.uint32), ref)
    finally:
        sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)


# ----------------------------------------------------- argument checks on GPU

def test_errors_launch_nothing(h):
    M, N, K = 4, 64, 512
    x, W = inputs(M, N, K, tag=95)
    xd, Wd = to_dev(x), to_dev(W.reshape(-1))
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    raw = sbb.qmm_run_raw
    assert raw(h, xd.data_ptr() + 4, Wd.data_ptr(), y.data_ptr(), M, N, K, s) == sbb.QMM_ERR_ALIGN
    assert raw(h, xd.data_ptr(), Wd.data_ptr(), y.data_ptr(), 33, N, K, s) == sbb.QMM_ERR_SHAPE
    assert raw(h, xd.data_ptr(), Wd.data_ptr(), y.data_ptr(), M, N, 300, s) == sbb.QMM_ERR_SHAPE
    assert raw(h, xd.data_ptr(), Wd.data_ptr(), xd.data_ptr() + 64, M, N, K, s) == sbb.QMM_ERR_OVERLAP
    sbb.qmm_set_shape(h, 9, 0, 0)  # 9 waves per workgroup is not a launch shape
    try:
        assert raw(h, xd.data_ptr(), Wd.data_ptr(), y.data_ptr(), M, N, K, s) == sbb.QMM_ERR_INVALID_ARG
    finally:
        sbb.qmm_set_shape(h, 0, 0, 0)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    assert raw(h, xd.data_ptr(), Wd.data_ptr(), y.data_ptr(), M, N, K, s) == sbb.QMM_OK
    torch.cuda.synchronize()
    yref, aref = oracle.qmm(x, W, N, K)
    check(y.cpu().numpy(), yref, aref, "after errors")


def test_create_reports_allocation_failure():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    os.environ["QMM_TEST_FAIL_ALLOC"] = "1"
    try:
        with pytest.raises(sbb.QmmError) as e:
            sbb.qmm_create(0)
        assert e.value.status == sbb.QMM_ERR_OOM
    finally:
        del os.environ["QMM_TEST_FAIL_ALLOC"]
    hh = sbb.qmm_create(0)
    sbb.qmm_destroy(hh)


@pytest.mark.parametrize("M,N,K", [(1, 5120, 5120), (16, 34816, 5120), (4, 5120, 17408)])
def test_launch_events_time_the_kernel(h, M, N, K):
    # events set with qmm_set_launch_events are recorded around the next
    # launch's kernel only: a positive duration, the same bits as an untimed
    # call, and the following call runs untimed again
    from skinny_bit_block_amd.events import EventPool
    x, W = inputs(M, N, K, tag=120 + M)
    xd, Wd = to_dev(x), to_dev(W.reshape(-1))
    y0 = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
    y1 = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
    sbb.qmm_run(h, xd, Wd, y0, M, N, K)
    pool = EventPool(1)
    try:
        sbb.qmm_set_launch_events(h, *pool.pairs[0])
        sbb.qmm_run(h, xd, Wd, y1, M, N, K)
        torch.cuda.synchronize()
        ms = pool.elapsed_ms(0)
        assert 0.0 < ms < 100.0
        # the weights cannot stream faster than 8 TB/s
        assert ms * 1e-3 >= sbb.qmm_weight_bytes(N, K) / 8e12
        assert torch.equal(y0, y1)
        sbb.qmm_run(h, xd, Wd, y1, M, N, K)  # untimed: the events were consumed
        torch.cuda.synchronize()
        assert pool.elapsed_ms(0) == ms
    finally:
        pool.close()

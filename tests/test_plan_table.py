"""Every launch-table shape plans at every row count 1..32 in every weight
format (4.5-bit super-blocks, block-scaled FP4, plain INT4), on a
planning-only handle: an entry whose shape does not fit LDS or the split-K
workspace would make the call fail with QMM_ERR_INVALID_ARG instead of reaching
the device check. CPU only."""
import pytest

import skinny_bit_block_amd as sbb

# the matrix shapes of the model pass (the table's shapes) and an unlisted one
SHAPES = [(5120, 5120), (34816, 5120), (5120, 17408), (151936, 5120), (2048, 2048)]
X, W, Y = 1 << 20, 1 << 32, 1 << 36  # aligned, disjoint fake device addresses


@pytest.fixture(scope="module")
def h():
    handle = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    yield handle
    sbb.qmm_destroy(handle)


@pytest.mark.parametrize("N,K", SHAPES)
def test_every_row_count_plans(h, N, K):
    for M in range(1, 33):
        p = sbb.qmm_query_plan(h, M, N, K)
        assert p["lds_bytes"] <= 160 * 1024
        assert p["splits"] >= p["wave_splits"] >= 1
        assert p["waves_per_wg"] % p["wave_splits"] == 0
        assert sbb.qmm_run_nvfp4_raw(h, X, W, 1.0, Y, M, N, K, None) == sbb.QMM_ERR_NO_DEVICE, \
            ("fp4", M, N, K)
        assert sbb.qmm_run_int4_raw(h, X, W, Y, M, N, K, None) == sbb.QMM_ERR_NO_DEVICE, \
            ("int4", M, N, K)


def test_kernel_switch_points(h):
    # one row: row-vector kernel on every table shape; two rows and more: tiled
    for N, K in SHAPES[:4]:
        assert sbb.qmm_query_plan(h, 1, N, K)["kernel"] == sbb.KERNEL_VECTOR
        for M in (2, 7, 16, 32):
            assert sbb.qmm_query_plan(h, M, N, K)["kernel"] == sbb.KERNEL_TILED

"""Property-based checks of the launch planner (planning-only handle, CPU):
for random row counts, matrix sizes, weight formats, expert slots and forced
launch overrides, a call is either rejected with one of the documented
argument statuses or planned so that
  - the waves, K slices and in-workgroup slices are consistent (every slice
    non-empty, the slices cover K, wave splits divide the waves; a forced
    wave split beyond the K slices leaves the extra wave slices idle inside
    one workgroup range),
  - the forced overrides are the ones used,
  - the LDS and the split-K workspace fit their limits,
  - the row-vector kernel only runs plain 4.5-bit calls of at most 8 rows,
  - and every load of the planned launch stays inside W and x (the host
    address replay of tests/test_address_sim.py).
"""
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import skinny_bit_block_amd as sbb  # noqa: E402
import test_address_sim as addr  # noqa: E402

LDS_MAX = 160 * 1024
WORKSPACE = 128 << 20
REJECT = {sbb.QMM_ERR_INVALID_ARG, sbb.QMM_ERR_SHAPE}


@pytest.fixture(scope="module")
def planner():
    h = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    yield h
    sbb.qmm_destroy(h)


calls = st.fixed_dictionaries({
    "M": st.integers(1, 32),
    "N": st.sampled_from([1, 2, 15, 16, 17, 31, 33, 100, 255, 257, 1000, 2047, 5120]),
    "nb": st.integers(1, 24),
    "fmt": st.sampled_from([sbb.FORMAT_KQUANT, sbb.FORMAT_KQUANT, sbb.FORMAT_NVFP4, sbb.FORMAT_INT4]),
    "slots": st.sampled_from([0, 0, 0, 1, 2, 5]),
    "kernel": st.sampled_from([sbb.KERNEL_AUTO, sbb.KERNEL_AUTO, sbb.KERNEL_VECTOR, sbb.KERNEL_TILED]),
    "waves": st.sampled_from([0, 0, 1, 2, 3, 4, 4, 6, 8, 8, 9]),
    "splits": st.sampled_from([0, 0, 0, 1, 2, 3, 5, 8, 13, 26]),
    "grid": st.sampled_from([0, 0, 0, 1, 2, 7, 300]),
    "wsplit": st.sampled_from([0, 0, 0, 1, 2, 2, 4, 9]),
})


@settings(max_examples=800, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(c=calls)
def test_plans_are_consistent_and_in_bounds(planner, c):
    M, N, nb, fmt = c["M"], c["N"], c["nb"], c["fmt"]
    K = 256 * nb
    slots = min(c["slots"], M) if fmt == sbb.FORMAT_KQUANT else 0
    try:
        try:  # an override can already be refused when it is set (more than 8 wave splits)
            sbb.qmm_set_kernel(planner, c["kernel"])
            sbb.qmm_set_shape(planner, c["waves"], c["splits"], c["grid"])
            sbb.qmm_set_wave_splits(planner, c["wsplit"])
            p = sbb.qmm_query_plan_format(planner, fmt, slots, M, N, K)
        except sbb.QmmError as e:
            assert e.status in REJECT, (c, e.status)
            hypothesis.event("rejected")
            return
    finally:
        sbb.qmm_set_kernel(planner, sbb.KERNEL_AUTO)
        sbb.qmm_set_shape(planner, 0, 0, 0)
        sbb.qmm_set_wave_splits(planner, 0)
    waves, splits, wsplit, nbs = p["waves_per_wg"], p["splits"], p["wave_splits"], p["blocks_per_split"]
    # shape of the work split
    assert 1 <= waves <= 8 and wsplit >= 1 and waves % wsplit == 0
    assert 1 <= splits <= nb
    assert nbs >= 1 and (splits - 1) * nbs < nb <= splits * nbs  # every slice non-empty, K covered
    grid_y = -(-splits // wsplit)
    if splits < wsplit:
        # a forced wave split beyond the K slices: one workgroup range, the
        # extra wave slices have no K work (each takes one empty step per tile)
        assert grid_y == 1
    assert p["grid_x"] >= 1
    # the overrides that were given are the ones used
    if c["waves"]:
        assert waves == c["waves"]
    if c["wsplit"]:
        assert wsplit == c["wsplit"]
    if c["splits"]:
        assert nbs == -(-nb // c["splits"])
    if c["grid"]:
        assert p["grid_x"] == c["grid"]
    # limits
    assert 0 < p["lds_bytes"] <= LDS_MAX
    assert p["workspace_bytes"] == (grid_y * M * N * 4 if grid_y > 1 else 0)
    assert p["workspace_bytes"] <= WORKSPACE
    # kernel choice
    if p["kernel"] == sbb.KERNEL_VECTOR:
        assert M <= 8 and fmt == sbb.FORMAT_KQUANT and slots == 0
        assert c["kernel"] != sbb.KERNEL_TILED
    else:
        assert c["kernel"] != sbb.KERNEL_VECTOR
    hypothesis.event("planned, %s" % ("split-K" if grid_y > 1 else "one range"))
    # every load of the launch in bounds, also as a persistent grid
    for m in sorted({1, M}) if slots else (M,):
        addr.replay(p, m, N, K, grids=(1, 5))

"""The C-ABI library loads, exports what include/qmm.h declares, and checks its
arguments on the host (no GPU needed: planning-only handles)."""
import ctypes
import os
import re

import pytest

import skinny_bit_block_amd as sbb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(header="qmm.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*\**\s*\b(\w+)\s*\(", src, re.M)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert "qmm_create" in names and "qmm_run" in names and "qmm_destroy" in names
    lib = ctypes.CDLL(sbb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(sbb.EXPORTS) == names


def test_every_header_is_exported():
    # every function any header under include/ declares is exported by the
    # library, and each header has a binding module listing exactly its names
    from skinny_bit_block_amd import gdn, probe
    lib = ctypes.CDLL(sbb.LIB_PATH)
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    listed = {"qmm.h": sbb.EXPORTS, "qmm_probe.h": probe.EXPORTS, "gdn.h": gdn.EXPORTS}
    assert set(headers) <= set(listed), headers
    for hname in headers:
        names = declared_functions(hname)
        assert names, hname
        for n in names:
            assert hasattr(lib, n), (hname, n)
        assert sorted(listed[hname]) == names, hname


def test_status_strings():
    for s in range(0, -8, -1):
        assert sbb.qmm_status_string(s).startswith("QMM_")
    assert "unknown" in sbb.qmm_status_string(-99)


def test_weight_bytes():
    assert sbb.qmm_weight_bytes(151936, 5120) == 437575680
    assert sbb.qmm_weight_bytes(1, 300) == 0


def test_no_device_here():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(sbb.QmmError) as e:
        sbb.qmm_create(0)
    assert e.value.status == sbb.QMM_ERR_NO_DEVICE


def test_destroy_null_is_ok():
    assert sbb.load().qmm_destroy(None) == 0


@pytest.fixture
def planner():
    h = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    yield h
    sbb.qmm_destroy(h)


def test_plans_for_every_workload(planner):
    cases = [(4, 2048, 2048)] + [(m, 34816, 5120) for m in (1, 2, 4, 7, 8, 9, 16)] + \
            [(m, 5120, 17408) for m in (1, 4, 8, 16)] + [(m, 151936, 5120) for m in (1, 7)] + \
            [(m, n, k) for m in (1, 4, 8, 16, 32) for n, k in ((5120, 5120), (34816, 5120),
                                                           (5120, 17408), (151936, 5120))]
    for M, N, K in cases:
        p = sbb.qmm_query_plan(planner, M, N, K)
        assert p["kernel"] == (sbb.KERNEL_TILED if M >= sbb.qmm_switch_point(planner, N, K)
                               else sbb.KERNEL_VECTOR)
        assert p["lds_bytes"] <= 160 * 1024
        nb = K // 256
        assert 1 <= p["splits"] <= nb and p["blocks_per_split"] * p["splits"] >= nb
        assert p["blocks_per_split"] * (p["splits"] - 1) < nb  # no empty slice
        ws, wsp = p["waves_per_wg"], p["wave_splits"]
        assert ws % wsp == 0 and p["splits"] >= wsp
        ranges = -(-p["splits"] // wsp)
        assert p["workspace_bytes"] == (ranges * M * N * 4 if ranges > 1 else 0)
        tiles = (N + 15) // 16
        assert p["grid_x"] == -(-tiles // (ws // wsp))


def test_switch_point_in_range(planner):
    for n, k in ((2048, 2048), (34816, 5120), (5120, 17408), (151936, 5120)):
        assert 1 <= sbb.qmm_switch_point(planner, n, k) <= 33


@pytest.mark.parametrize("M,N,K,status", [
    (0, 16, 256, sbb.QMM_ERR_SHAPE), (33, 16, 256, sbb.QMM_ERR_SHAPE),
    (1, 0, 256, sbb.QMM_ERR_SHAPE), (1, 16, 0, sbb.QMM_ERR_SHAPE),
    (1, 16, 300, sbb.QMM_ERR_SHAPE), (1, 16, 128, sbb.QMM_ERR_SHAPE),
])
def test_shape_errors(planner, M, N, K, status):
    with pytest.raises(sbb.QmmError) as e:
        sbb.qmm_query_plan(planner, M, N, K)
    assert e.value.status == status
    # qmm_run checks before touching anything; fake aligned pointers are never dereferenced
    assert sbb.qmm_run_raw(planner, 0x10000, 0x20000000, 0x40000000, M, N, K, 0) == status


def test_run_argument_checks(planner):
    run = sbb.qmm_run_raw
    assert run(None, 0x10000, 0x20000000, 0x40000000, 1, 16, 256, 0) == sbb.QMM_ERR_INVALID_ARG
    assert run(planner, 0, 0x20000000, 0x40000000, 1, 16, 256, 0) == sbb.QMM_ERR_INVALID_ARG
    assert run(planner, 0x10000, 0, 0x40000000, 1, 16, 256, 0) == sbb.QMM_ERR_INVALID_ARG
    assert run(planner, 0x10000, 0x20000000, 0, 1, 16, 256, 0) == sbb.QMM_ERR_INVALID_ARG
    assert run(planner, 0x10004, 0x20000000, 0x40000000, 1, 16, 256, 0) == sbb.QMM_ERR_ALIGN
    assert run(planner, 0x10000, 0x20000008, 0x40000000, 1, 16, 256, 0) == sbb.QMM_ERR_ALIGN
    assert run(planner, 0x10000, 0x20000000, 0x40000002, 1, 16, 256, 0) == sbb.QMM_ERR_ALIGN
    # y overlapping x or W
    assert run(planner, 0x10000, 0x20000000, 0x10000 + 512, 1, 16, 256, 0) == sbb.QMM_ERR_OVERLAP
    assert run(planner, 0x10000, 0x20000000, 0x20000000 + 144, 1, 16, 256, 0) == sbb.QMM_ERR_OVERLAP
    # valid arguments on a planning-only handle: nothing can run
    assert run(planner, 0x10000, 0x20000000, 0x40000000, 1, 16, 256, 0) == sbb.QMM_ERR_NO_DEVICE


def test_overrides(planner):
    sbb.qmm_set_kernel(planner, sbb.KERNEL_TILED)
    assert sbb.qmm_query_plan(planner, 1, 2048, 2048)["kernel"] == sbb.KERNEL_TILED
    assert sbb.qmm_query_plan(planner, 8, 2048, 2048)["kernel"] == sbb.KERNEL_TILED
    sbb.qmm_set_kernel(planner, sbb.KERNEL_VECTOR)
    assert sbb.qmm_query_plan(planner, 8, 2048, 2048)["kernel"] == sbb.KERNEL_VECTOR
    with pytest.raises(sbb.QmmError) as e:  # the row-vector kernel stops at 8 rows
        sbb.qmm_query_plan(planner, 9, 2048, 2048)
    assert e.value.status == sbb.QMM_ERR_INVALID_ARG
    sbb.qmm_set_kernel(planner, sbb.KERNEL_AUTO)
    sbb.qmm_set_shape(planner, 4, 2, 40)
    p = sbb.qmm_query_plan(planner, 4, 2048, 2048)
    assert (p["waves_per_wg"], p["splits"], p["grid_x"]) == (4, 2, 40)
    sbb.qmm_set_shape(planner, 4, 2, 1)  # one workgroup walks all 128 tiles of a slice
    assert sbb.qmm_query_plan(planner, 4, 2048, 2048)["grid_x"] == 1
    sbb.qmm_set_shape(planner, 9, 0, 0)  # at most 8 waves per workgroup
    with pytest.raises(sbb.QmmError):
        sbb.qmm_query_plan(planner, 4, 2048, 2048)
    sbb.qmm_set_shape(planner, 0, 9, 0)  # 9 slices of an 8-block K
    with pytest.raises(sbb.QmmError):
        sbb.qmm_query_plan(planner, 4, 2048, 2048)
    sbb.qmm_set_shape(planner, 0, 0, 0)
    with pytest.raises(sbb.QmmError):
        sbb.qmm_set_kernel(planner, 7)
    # slices reduced inside a workgroup
    sbb.qmm_set_shape(planner, 4, 4, 0)
    sbb.qmm_set_wave_splits(planner, 2)
    p = sbb.qmm_query_plan(planner, 4, 2048, 2048)
    assert (p["wave_splits"], p["splits"]) == (2, 4) and p["workspace_bytes"] == 2 * 4 * 2048 * 4
    sbb.qmm_set_wave_splits(planner, 4)
    p = sbb.qmm_query_plan(planner, 4, 2048, 2048)
    assert p["wave_splits"] == 4 and p["workspace_bytes"] == 0 and p["grid_x"] == 128
    sbb.qmm_set_wave_splits(planner, 3)  # 4 waves are not a multiple of 3
    with pytest.raises(sbb.QmmError):
        sbb.qmm_query_plan(planner, 4, 2048, 2048)
    sbb.qmm_set_shape(planner, 6, 2, 0)  # fewer slices than wave splits
    with pytest.raises(sbb.QmmError):
        sbb.qmm_query_plan(planner, 4, 2048, 2048)
    with pytest.raises(sbb.QmmError):
        sbb.qmm_set_wave_splits(planner, 9)
    sbb.qmm_set_wave_splits(planner, 0)
    sbb.qmm_set_shape(planner, 0, 0, 0)


def test_run_ids_argument_checks(planner):
    run = sbb.qmm_run_ids_raw
    ok = (0x10000, 0x20000000, 0x30000000, 8, 0x40000000, 4, 16, 256, 0)
    assert run(None, *ok) == sbb.QMM_ERR_INVALID_ARG
    assert run(planner, 0x10000, 0x20000000, 0, 8, 0x40000000, 4, 16, 256, 0) == sbb.QMM_ERR_INVALID_ARG
    assert run(planner, 0x10000, 0x20000000, 0x30000000, 0, 0x40000000, 4, 16, 256, 0) == sbb.QMM_ERR_INVALID_ARG
    assert run(planner, 0x10000, 0x20000000, 0x30000002, 8, 0x40000000, 4, 16, 256, 0) == sbb.QMM_ERR_ALIGN
    assert run(planner, 0x10000, 0x20000000, 0x30000000, 8, 0x40000000, 33, 16, 256, 0) == sbb.QMM_ERR_SHAPE
    # y over the ids, over the last expert's bytes
    assert run(planner, 0x10000, 0x20000000, 0x40000000 + 8, 8, 0x40000000, 4, 16, 256, 0) == sbb.QMM_ERR_OVERLAP
    assert run(planner, 0x10000, 0x20000000, 0x30000000, 8, 0x20000000 + 7 * 16 * 144, 4, 16, 256, 0) == sbb.QMM_ERR_OVERLAP
    assert run(planner, *ok) == sbb.QMM_ERR_NO_DEVICE


def test_probe_argument_checks():
    # host-side checks of the probes, before any device call (no GPU needed)
    from skinny_bit_block_amd import probe
    lib = probe._lib()
    vp = ctypes.c_void_p
    khz = ctypes.c_int(0)
    fake = vp(0x10000)  # never dereferenced: every call below fails its checks first
    assert lib.qmm_probe_read(None, 16, 1, 64, fake, None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_read(fake, 16, 0, 64, fake, None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_read(fake, 16, 1, 96, fake, None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_read(vp(0x10008), 16, 1, 64, fake, None) == sbb.QMM_ERR_ALIGN
    assert lib.qmm_probe_read(fake, 24, 1, 64, fake, None) == sbb.QMM_ERR_ALIGN
    assert lib.qmm_probe_empty(0, None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_clock(None, 1, 1, ctypes.byref(khz), None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_clock(fake, 1, 1, None, None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_clock(fake, 0, 1, ctypes.byref(khz), None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_clock(fake, (1 << 20) + 1, 1, ctypes.byref(khz), None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_clock(fake, 1, 0, ctypes.byref(khz), None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_clock(fake, 1, (1 << 26) + 1, ctypes.byref(khz), None) == sbb.QMM_ERR_INVALID_ARG
    assert lib.qmm_probe_clock(vp(0x10004), 1, 1, ctypes.byref(khz), None) == sbb.QMM_ERR_ALIGN

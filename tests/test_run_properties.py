"""Property-based test of the product entry points' pointer rules (CPU, no
GPU: fake addresses that are never dereferenced). Buffers are placed at random,
often on top of one another; every entry point must return QMM_ERR_ALIGN for
a misaligned pointer (x and W 16-byte, y and ids 4-byte aligned), else
QMM_ERR_OVERLAP exactly when y meets x, the weights or the ids (x and the
weights may share memory), else pass its checks and stop at the device
(QMM_ERR_NO_DEVICE on a planning-only handle or with no GPU). The extents
are the ones include/qmm.h documents: x M*K*4 bytes, y M*N*4, W N*K/256*144
(E matrices of that size for the expert-indexed call), ids M*4."""
import ctypes

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import skinny_bit_block_amd as sbb  # noqa: E402

BASE = 1 << 36
KINDS = ["run", "static", "nvfp4", "int4", "ids"]


@pytest.fixture(scope="module")
def planner():
    h = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    yield h
    sbb.qmm_destroy(h)


def meets(a, na, b, nb):
    return a < b + nb and b < a + na


@settings(max_examples=600, deadline=None, derandomize=True)
@given(data=st.data())
def test_pointer_rules(planner, data):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: qmm_run_static would reach the device")
    kind = data.draw(st.sampled_from(KINDS))
    M, N = data.draw(st.integers(1, 32)), data.draw(st.integers(1, 3000))
    K = 256 * data.draw(st.integers(1, 20))
    E = data.draw(st.integers(1, 4)) if kind == "ids" else 1
    ext = {"x": M * K * 4, "W": E * sbb.qmm_weight_bytes(N, K), "y": M * N * 4}
    if kind == "ids":
        ext["ids"] = M * 4
    names = list(ext)
    slot = {n: data.draw(st.integers(0, 7)) for n in names}
    off = {n: 16 * data.draw(st.integers(0, 1 << 15)) for n in names}
    ptr = {n: BASE + slot[n] * (1 << 22) + off[n] for n in names}
    mis = data.draw(st.sampled_from(names)) if data.draw(st.integers(0, 7)) == 0 else None
    if mis:
        ptr[mis] += data.draw(st.sampled_from([2, 4, 8] if mis in ("x", "W") else [1, 2]))
    lib = sbb.load()
    vp = ctypes.c_void_p
    if kind == "run":
        got = lib.qmm_run(planner, vp(ptr["x"]), vp(ptr["W"]), vp(ptr["y"]), M, N, K, None)
    elif kind == "static":
        got = sbb.qmm_run_static_raw(vp(ptr["x"]), vp(ptr["W"]), vp(ptr["y"]), M, N, K, None)
    elif kind == "nvfp4":
        got = sbb.qmm_run_nvfp4_raw(planner, vp(ptr["x"]), vp(ptr["W"]), 0.5, vp(ptr["y"]), M, N, K, None)
    elif kind == "int4":
        got = sbb.qmm_run_int4_raw(planner, vp(ptr["x"]), vp(ptr["W"]), vp(ptr["y"]), M, N, K, None)
    else:
        got = sbb.qmm_run_ids_raw(planner, vp(ptr["x"]), vp(ptr["W"]), vp(ptr["ids"]), E,
                                  vp(ptr["y"]), M, N, K, None)
    aligned = all(ptr[n] % (16 if n in ("x", "W") else 4) == 0 for n in names)
    if not aligned:
        hypothesis.event("misaligned")
        assert got == sbb.QMM_ERR_ALIGN, (kind, M, N, K, ptr, got)
        return
    clash = any(meets(ptr["y"], ext["y"], ptr[n], ext[n]) for n in names if n != "y")
    hypothesis.event("overlap" if clash else "disjoint")
    assert got == (sbb.QMM_ERR_OVERLAP if clash else sbb.QMM_ERR_NO_DEVICE), (kind, M, N, K, ptr, got)

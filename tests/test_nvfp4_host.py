"""Host side of the block-scaled FP4 path: the repack into the library's
144-byte groups, read back with a reader written from the layout stated in
include/qmm.h. CPU only (the repack is a host function of the library)."""
import numpy as np
import pytest

import skinny_bit_block_amd as sbb
import synth


def _usual_code(elems, n, k):
    return (int(elems[n, k // 2]) >> (4 * (k % 2))) & 0xF


def _group_code(groups, n, k):
    b, e = divmod(k, 256)
    c, r = divmod(e, 64)
    byte = int(groups[n, b * 144 + 16 + 32 * c + r % 32])
    return byte & 0xF if r < 32 else byte >> 4


@pytest.mark.parametrize("N,K", [(1, 256), (3, 512), (5, 1280)])
def test_repack_layout(N, K):
    elems, scales = synth.nvfp4(N, K, tensor=21)
    groups = sbb.qmm_nvfp4_repack(elems, scales, N, K)
    assert groups.shape == (N, K // 256 * 144)
    assert groups.size == sbb.qmm_weight_bytes(N, K)
    for n in range(N):
        for b in range(K // 256):
            assert np.array_equal(groups[n, b * 144:b * 144 + 16], scales[n, 16 * b:16 * b + 16])
        for k in range(K):
            assert _group_code(groups, n, k) == _usual_code(elems, n, k), (n, k)


def test_repack_rejects_bad_shapes():
    elems, scales = synth.nvfp4(2, 384, tensor=22)
    with pytest.raises(sbb.QmmError) as e:
        sbb.qmm_nvfp4_repack(elems, scales, 2, 384)
    assert e.value.status == sbb.QMM_ERR_SHAPE
    with pytest.raises(ValueError):
        sbb.qmm_nvfp4_repack(elems[:1], scales, 2, 384)


def test_run_nvfp4_argument_checks():
    h = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    try:
        # null pointers and a non-finite tensor scale are rejected before any launch
        assert sbb.qmm_run_nvfp4_raw(h, None, None, 1.0, None, 1, 16, 256, None) == \
            sbb.QMM_ERR_INVALID_ARG
        assert sbb.qmm_run_nvfp4_raw(h, 16, 16, float("inf"), 4096, 1, 16, 256, None) == \
            sbb.QMM_ERR_INVALID_ARG
        # shape and alignment before the device check
        assert sbb.qmm_run_nvfp4_raw(h, 16, 16, 1.0, 4096, 1, 16, 300, None) == sbb.QMM_ERR_SHAPE
        assert sbb.qmm_run_nvfp4_raw(h, 8, 16, 1.0, 4096, 1, 16, 256, None) == sbb.QMM_ERR_ALIGN
        # a planning-only handle plans but launches nothing
        assert sbb.qmm_run_nvfp4_raw(h, 16, 1 << 20, 1.0, 1 << 30, 1, 16, 256, None) == \
            sbb.QMM_ERR_NO_DEVICE
    finally:
        sbb.qmm_destroy(h)

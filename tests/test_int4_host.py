"""Host side of the plain INT4 path: the repack into the library's 144-byte
groups, read back with a reader written from the layout stated in
include/qmm.h. CPU only (the repack is a host function of the library)."""
import numpy as np
import pytest

import skinny_bit_block_amd as sbb
import synth


def _usual_code(codes, n, k):
    return (int(codes[n, k // 2]) >> (4 * (k % 2))) & 0xF


def _group_code(groups, n, k):
    # the stored code is offset by 8: two's complement q -> q + 8 (top bit flipped)
    b, e = divmod(k, 256)
    c, r = divmod(e, 64)
    byte = int(groups[n, b * 144 + 16 + 32 * c + r % 32])
    return ((byte & 0xF) if r < 32 else (byte >> 4)) ^ 0x8


@pytest.mark.parametrize("N,K", [(1, 256), (3, 512), (5, 1280)])
def test_repack_layout(N, K):
    codes, scales = synth.int4(N, K, tensor=31)
    groups = sbb.qmm_int4_repack(codes, scales, N, K)
    assert groups.shape == (N, K // 256 * 144)
    assert groups.size == sbb.qmm_weight_bytes(N, K)
    for n in range(N):
        for b in range(K // 256):
            g = groups[n, b * 144:b * 144 + 16]
            assert int(g[0]) | int(g[1]) << 8 == int(scales[n, 2 * b])
            assert int(g[2]) | int(g[3]) << 8 == int(scales[n, 2 * b + 1])
            assert not g[4:].any()
        for k in range(K):
            assert _group_code(groups, n, k) == _usual_code(codes, n, k), (n, k)


def test_repack_rejects_bad_shapes():
    codes, scales = synth.int4(2, 384, tensor=32)
    with pytest.raises(sbb.QmmError) as e:
        sbb.qmm_int4_repack(codes, scales, 2, 384)
    assert e.value.status == sbb.QMM_ERR_SHAPE
    with pytest.raises(ValueError):
        sbb.qmm_int4_repack(codes[:1], scales, 2, 384)


def test_run_int4_argument_checks():
    h = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    try:
        assert sbb.qmm_run_int4_raw(h, None, None, None, 1, 16, 256, None) == \
            sbb.QMM_ERR_INVALID_ARG
        # shape and alignment before the device check
        assert sbb.qmm_run_int4_raw(h, 16, 16, 4096, 1, 16, 300, None) == sbb.QMM_ERR_SHAPE
        assert sbb.qmm_run_int4_raw(h, 16, 16, 4096, 33, 16, 256, None) == sbb.QMM_ERR_SHAPE
        assert sbb.qmm_run_int4_raw(h, 8, 16, 4096, 1, 16, 256, None) == sbb.QMM_ERR_ALIGN
        # y overlapping the weights
        assert sbb.qmm_run_int4_raw(h, 1 << 24, 1 << 20, 1 << 20, 1, 16, 256, None) == \
            sbb.QMM_ERR_OVERLAP
        # a planning-only handle plans but launches nothing
        assert sbb.qmm_run_int4_raw(h, 16, 1 << 20, 1 << 30, 1, 16, 256, None) == \
            sbb.QMM_ERR_NO_DEVICE
    finally:
        sbb.qmm_destroy(h)

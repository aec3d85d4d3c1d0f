"""Pins of the block-scaled FP4 oracle (oracle/nvfp4.py) to the format's
public definitions: the E2M1 value table, torch's own E4M3 decoding, hand-built
rows, position probes and closed forms. CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import nvfp4 as fp4

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "nvfp4.txt")


def _golden():
    sec, out = None, {"e2m1": {}, "e4m3": {}, "row": {}}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("["):
            sec = line.strip("[]")
            continue
        key, *vals = line.split()
        if sec in ("e2m1", "e4m3"):
            out[sec][int(key, 16)] = float(vals[0])
        else:
            out["row"][key] = vals
    return out


G = _golden()


def test_e2m1_spec_table():
    assert len(G["e2m1"]) == 16
    for code, v in G["e2m1"].items():
        got = fp4.e2m1_value(code)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), code


def test_e4m3_named_points():
    for code, v in G["e4m3"].items():
        assert fp4.e4m3_value(code) == v, hex(code)
    assert math.isnan(fp4.e4m3_value(0x7F)) and math.isnan(fp4.e4m3_value(0xFF))


def test_e4m3_every_code_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for code in range(256):
        got, want = fp4.e4m3_value(code), float(ref[code])
        if math.isnan(want):
            assert math.isnan(got), hex(code)
        else:
            assert got == want, hex(code)


def test_hand_built_row():
    r = G["row"]
    elems = np.array([[int(b, 16) for b in r["elems"]]], dtype=np.uint8)
    scales = np.array([[int(b, 16) for b in r["scales"]]], dtype=np.uint8)
    w = fp4.dequant_rows(elems, scales, float(r["tensor"][0]), 32)[0]
    want = np.array([float(v) for v in r["w"]])
    assert np.array_equal(w, want)


@pytest.mark.parametrize("pos", [0, 1, 14, 15, 16, 17, 30, 31, 62, 63])
def test_element_position_one_hot(pos):
    K = 64
    elems = np.zeros((1, K // 2), dtype=np.uint8)
    elems[0, pos // 2] = 0x2 << (4 * (pos % 2))  # code 0x2 (= 1.0) at element pos
    scales = np.full((1, K // 16), 0x38, dtype=np.uint8)  # 1.0
    w = fp4.dequant_rows(elems, scales, 1.0, K)[0]
    assert w[pos] == 1.0 and np.count_nonzero(w) == 1


@pytest.mark.parametrize("j", [0, 1, 3])
def test_scale_covers_its_sixteen(j):
    K = 64
    elems = np.full((1, K // 2), 0x22, dtype=np.uint8)  # every element 1.0
    scales = np.full((1, K // 16), 0x38, dtype=np.uint8)
    scales[0, j] = 0x40  # 2.0
    w = fp4.dequant_rows(elems, scales, 1.0, K)[0]
    want = np.ones(K)
    want[16 * j:16 * j + 16] = 2.0
    assert np.array_equal(w, want)


def test_zero_and_subnormal_scales():
    elems = np.full((1, 8), 0x77, dtype=np.uint8)  # 6.0 everywhere
    w0 = fp4.dequant_rows(elems, np.array([[0x00]], dtype=np.uint8), 1.0, 16)[0]
    w1 = fp4.dequant_rows(elems, np.array([[0x01]], dtype=np.uint8), 1.0, 16)[0]
    assert not w0.any()
    assert np.all(w1 == 6.0 * 2.0 ** -9)


def test_product_brute_force():
    M, N, K = 3, 5, 48
    elems, scales = synth.nvfp4(N, K, tensor=11)
    x = synth.acts(M, K, tensor=12)
    y, a = fp4.qmm_nvfp4(x, elems, scales, 0.75, N, K)
    for m in range(M):
        for n in range(N):
            s = sa = 0.0
            for k in range(K):
                code = (elems[n, k // 2] >> (4 * (k % 2))) & 0xF
                w = 0.75 * fp4.e4m3_value(scales[n, k // 16]) * fp4.e2m1_value(code)
                s += float(x[m, k]) * w
                sa += abs(float(x[m, k]) * w)
            assert math.isclose(y[m, n], s, rel_tol=1e-12, abs_tol=1e-12)
            assert math.isclose(a[m, n], sa, rel_tol=1e-12, abs_tol=1e-12)


def test_tensor_scale_is_linear():
    N, K = 7, 256
    elems, scales = synth.nvfp4(N, K, tensor=13)
    x = synth.acts(2, K, tensor=14)
    y1, _ = fp4.qmm_nvfp4(x, elems, scales, 1.0, N, K)
    y4, _ = fp4.qmm_nvfp4(x, elems, scales, 4.0, N, K)
    assert np.array_equal(y4, 4.0 * y1)


def test_rows_subset_matches_full():
    N, K = 9, 512
    elems, scales = synth.nvfp4(N, K, tensor=15)
    x = synth.acts(4, K, tensor=16)
    y, a = fp4.qmm_nvfp4(x, elems, scales, 1.5, N, K)
    ys, as_ = fp4.qmm_nvfp4(x, elems, scales, 1.5, N, K, rows=[8, 0, 3])
    assert np.array_equal(ys, y[:, [8, 0, 3]]) and np.array_equal(as_, a[:, [8, 0, 3]])


def test_rejects_bad_shapes():
    e, s = synth.nvfp4(2, 32, tensor=17)
    with pytest.raises(ValueError):
        fp4.dequant_rows(e, s, 1.0, 48)
    with pytest.raises(ValueError):
        fp4.dequant_rows(e, s[:, :1], 1.0, 32)
    with pytest.raises(TypeError):
        fp4.dequant_rows(e.astype(np.int16), s, 1.0, 32)


def test_generator_fields():
    e, s = synth.nvfp4(64, 1024, tensor=18)
    assert e.shape == (64, 512) and s.shape == (64, 64)
    assert (s & 0x80).max() == 0 and (s >> 3).max() <= 14  # no sign, no NaN code
    assert len(np.unique(e)) > 200

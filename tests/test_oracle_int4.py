"""Pins of the plain INT4 oracle (oracle/int4.py) to the format's definition:
the two's-complement table, hand-decoded binary16 values and numpy's own
binary16 decoding, a hand-built row, position probes, brute force and exact
zeros. CPU only."""
import os

import numpy as np
import pytest

import synth
from oracle import int4

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "int4.txt")


def _golden():
    sec, out = None, {"int4": {}, "f16": {}, "row": {}}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("["):
            sec = line.strip("[]")
            continue
        key, *vals = line.split()
        if sec in ("int4", "f16"):
            out[sec][int(key, 16)] = float(vals[0])
        else:
            out["row"][key] = vals
    return out


G = _golden()


def test_twos_complement_table():
    assert len(G["int4"]) == 16
    for code, v in G["int4"].items():
        assert int4.int4_value(code) == v


def test_f16_hand_decoded_points():
    for bits, v in G["f16"].items():
        assert int4.f16_value(bits) == v, hex(bits)


def test_f16_every_pattern_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([int4.f16_value(b) for b in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of the zeros too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _hand_row():
    K = 256
    codes = np.zeros((1, K // 2), dtype=np.uint8)
    for item in G["row"]["bytes"]:
        i, b = item.split(":")
        codes[0, int(i)] = int(b, 16)
    scales = np.array([[int(s, 16) for s in G["row"]["scales"]]], dtype=np.uint16)
    w = np.zeros(K)
    for item in G["row"]["w"]:
        k, v = item.split(":")
        w[int(k)] = float(v)
    return codes, scales, w


def test_hand_built_row():
    codes, scales, w = _hand_row()
    got = int4.dequant_rows(codes, scales, 256)[0]
    assert np.array_equal(got, w)


def test_hand_built_row_product():
    codes, scales, w = _hand_row()
    x = np.linspace(-1.0, 1.0, 256)[None, :]
    y, a = int4.qmm_int4(x, codes, scales, 1, 256)
    assert y[0, 0] == pytest.approx(float(np.sum(w * x[0])), rel=1e-15, abs=1e-15)
    assert a[0, 0] == pytest.approx(float(np.sum(np.abs(w * x[0]))), rel=1e-15)


@pytest.mark.parametrize("k", [0, 1, 2, 127, 128, 129, 255, 256, 383, 511])
def test_one_hot_code_position(k):
    # element k = 1 (its nibble: low for even k), everything else 0, scales 1
    K = 512
    codes = np.zeros((2, K // 2), dtype=np.uint8)
    codes[1, k // 2] = 1 << (4 * (k % 2))
    scales = np.full((2, K // 128), 0x3C00, dtype=np.uint16)
    w = int4.dequant_rows(codes, scales, K)
    assert np.count_nonzero(w) == 1 and w[1, k] == 1.0


@pytest.mark.parametrize("j", [0, 1, 2, 3])
def test_one_hot_scale_position(j):
    # every code 1; scale j = 2.0, the others 1.0: weight 2 exactly on 128j..128j+127
    K = 512
    codes = np.full((1, K // 2), 0x11, dtype=np.uint8)
    scales = np.full((1, K // 128), 0x3C00, dtype=np.uint16)
    scales[0, j] = 0x4000
    w = int4.dequant_rows(codes, scales, K)[0]
    expect = np.ones(K)
    expect[128 * j:128 * j + 128] = 2.0
    assert np.array_equal(w, expect)


def test_brute_force_small():
    # every element decoded one at a time from its byte, nibble and scale
    N, K, M = 3, 256, 2
    codes, scales = synth.int4(N, K, tensor=7, seed=11)
    x = synth.acts(M, K, tensor=8, seed=11).astype(np.float64)
    y, a = int4.qmm_int4(x, codes, scales, N, K)
    for m in range(M):
        for n in range(N):
            s = sa = 0.0
            for k in range(K):
                byte = int(codes[n, k // 2])
                nib = (byte >> 4) if k % 2 else (byte & 0xF)
                q = nib - 16 if nib >= 8 else nib
                sc = int4.f16_value(int(scales[n, k // 128]))
                s += x[m, k] * sc * q
                sa += abs(x[m, k] * sc * q)
            assert y[m, n] == pytest.approx(s, rel=1e-12, abs=1e-12)
            assert a[m, n] == pytest.approx(sa, rel=1e-12)


def test_zero_codes_give_exact_zero():
    N, K = 4, 256
    _, scales = synth.int4(N, K, tensor=9, seed=3)
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    x = synth.acts(2, K, tensor=10, seed=3)
    y, a = int4.qmm_int4(x, codes, scales, N, K)
    assert np.all(y == 0.0) and np.all(a == 0.0)


def test_negation_symmetry():
    # code c and its negation (two's complement, c != -8) give opposite weights
    K = 128
    c = np.arange(1, 8, dtype=np.uint8)
    neg = (16 - c) & 0xF
    assert all(int4.int4_value(a) == -int4.int4_value(b) for a, b in zip(c, neg))
    codes = np.zeros((2, K // 2), dtype=np.uint8)
    codes[0, :7] = c
    codes[1, :7] = neg
    scales = np.full((2, 1), 0x3A00, dtype=np.uint16)
    w = int4.dequant_rows(codes, scales, K)
    assert np.array_equal(w[0], -w[1])


def test_rows_subset_matches_full():
    N, K = 40, 384
    codes, scales = synth.int4(N, K, tensor=12, seed=4)
    x = synth.acts(3, K, tensor=13, seed=4)
    y, a = int4.qmm_int4(x, codes, scales, N, K)
    rows = [0, 7, 39, 13]
    ys, as_ = int4.qmm_int4(x, codes, scales, N, K, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(as_, a[:, rows])


def test_rejects_bad_shapes():
    codes = np.zeros((2, 64), dtype=np.uint8)
    scales = np.zeros((2, 1), dtype=np.uint16)
    with pytest.raises(ValueError):
        int4.dequant_rows(codes, scales, 100)
    with pytest.raises(TypeError):
        int4.dequant_rows(codes, scales.astype(np.uint8), 128)
    with pytest.raises(ValueError):
        int4.dequant_rows(codes[:, :32], scales, 128)

"""Pins of the binary64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: the expected values come from
hand-built blocks (tests/golden/blocks.txt), an exact rational evaluator with
its own decoder (tests/exact_ref.py), numpy's binary16, closed forms and
invariants.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
import exact_ref
import goldens

ULP_BOUND = 2.0 ** -53


def test_f16_decode_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and the subnormal range
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0
    assert oracle.f16_to_f64(0x0001) == 2.0 ** -24
    assert oracle.f16_to_f64(0x03FF) == 1023 * 2.0 ** -24
    assert oracle.f16_to_f64(0x0400) == 2.0 ** -14


@pytest.mark.parametrize("name", ["scales_low", "scales_high_bits", "subnormal_scales",
                                  "negative_scales", "largest_d"])
def test_hand_built_blocks(name):
    spec = goldens.blocks()[name]
    blk = goldens.block_bytes(spec)
    w = oracle.dequant_block(blk)
    for j in range(8):
        assert np.all(w[32 * j:32 * j + 32] == spec["expect"][j]), (name, j, w[32 * j])


def test_hand_built_scale_fields():
    g = goldens.blocks()
    blk = goldens.block_bytes(g["scales_high_bits"])
    got = [oracle.scale_min(blk, j) for j in range(8)]
    assert got == [(0, 0)] * 4 + [(16, 63), (32, 48), (48, 32), (63, 17)]
    blk = goldens.block_bytes(g["scales_low"])
    assert [oracle.scale_min(blk, j) for j in range(8)] == [(j + 1, j) for j in range(8)]


def _quant_order_block(name, low, high):
    spec = goldens.blocks()[name]
    qs = bytes((low(i) & 15) | ((high(i) & 15) << 4) for i in range(128))
    return goldens.block_bytes(spec, qs)


def test_quant_order_a():
    blk = _quant_order_block("quant_order_a", lambda i: i & 15, lambda i: i >> 4)
    w = oracle.dequant_block(blk)
    for c in range(4):
        for r in range(64):
            expect = (r & 15) if r < 32 else 2 * c + (r - 32) // 16
            assert w[64 * c + r] == expect, (c, r)


def test_quant_order_b():
    blk = _quant_order_block("quant_order_b", lambda i: i >> 3, lambda i: 3 * i)
    w = oracle.dequant_block(blk)
    for c in range(4):
        for r in range(64):
            expect = (4 * c + r // 8) if r < 32 else (3 * (r - 32)) & 15
            assert w[64 * c + r] == expect, (c, r)


def test_random_blocks_match_exact_decoder():
    W = synth.weights(3, 1024, tensor=91, seed=5)
    for n in range(3):
        for b in range(4):
            blk = W[n, b * 144:(b + 1) * 144]
            ref = exact_ref.block_weights(blk.tobytes())
            got = oracle.dequant_block(blk)
            # w is exact in binary64 (d*sc*q and dmin*m span at most 51 bits)
            assert [Fraction(float(v)) for v in got] == ref


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 256, 1), (3, 4, 512, 2), (2, 3, 256, 3)])
def test_product_within_rounding_of_exact(M, N, K, seed):
    W = synth.weights(N, K, tensor=100 + seed, seed=seed)
    x = synth.acts(M, K, tensor=200 + seed, seed=seed)
    y, a = oracle.qmm(x, W, N, K)
    ye, ae = exact_ref.product(x, W, N, K)
    for m in range(M):
        for n in range(N):
            bound = (K + 2) * ULP_BOUND * float(ae[m][n])
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= Fraction(bound), (m, n)
            assert abs(a[m, n] - float(ae[m][n])) <= bound


def test_one_hot_reads_out_weights():
    N, K = 5, 512
    W = synth.weights(N, K, tensor=7, seed=11)
    wex = exact_ref.matrix_weights(W.tobytes(), N, K)
    for k in [0, 31, 32, 63, 64, 255, 256, 300, 511]:
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        y, a = oracle.qmm(x, W, N, K)
        assert [Fraction(v) for v in y[0]] == [wex[n][k] for n in range(N)]
        assert [Fraction(v) for v in a[0]] == [abs(wex[n][k]) for n in range(N)]


def test_all_ones_closed_form():
    N, K = 4, 512
    W = synth.weights(N, K, tensor=8, seed=12)
    y, a = oracle.qmm(np.ones((1, K), dtype=np.float32), W, N, K)
    Wb = W.tobytes()
    for n in range(N):
        total = Fraction(0)
        for b in range(K // 256):
            blk = Wb[(n * (K // 256) + b) * 144:(n * (K // 256) + b + 1) * 144]
            d = exact_ref.f16_exact(blk[0] | blk[1] << 8)
            dmin = exact_ref.f16_exact(blk[2] | blk[3] << 8)
            sm = exact_ref.scales_mins(blk[4:16])
            q = exact_ref.quants(blk[16:])
            for j in range(8):
                total += d * sm[j][0] * sum(q[32 * j:32 * j + 32]) - 32 * dmin * sm[j][1]
        assert abs(Fraction(y[0, n]) - total) <= Fraction((K + 2) * ULP_BOUND * a[0, n])


def test_zero_scales_give_exact_zero():
    N, K, M = 6, 768, 3
    x = synth.acts(M, K, tensor=9, seed=13)
    W = synth.weights(N, K, tensor=10, seed=13).copy()
    Wz = W.reshape(N, K // 256, 144).copy()
    Wz[:, :, 0:4] = 0  # d = dmin = 0
    y, _ = oracle.qmm(x, Wz.reshape(N, -1), N, K)
    assert np.all(y == 0.0)
    Wz = W.reshape(N, K // 256, 144).copy()
    Wz[:, :, 4:16] = 0  # every sc = m = 0
    y, _ = oracle.qmm(x, Wz.reshape(N, -1), N, K)
    assert np.all(y == 0.0)


def test_unit_scales_reduce_to_integer_matmul():
    # d = 1, sc = 1, dmin = 0: w = q, so y = x . q^T (numpy matmul in binary64).
    N, K, M = 7, 512, 3
    x = synth.acts(M, K, tensor=11, seed=14)
    Wb = synth.weights(N, K, tensor=12, seed=14).reshape(N, K // 256, 144).copy()
    Wb[:, :, 0:2] = [0x00, 0x3C]
    Wb[:, :, 2:4] = 0
    Wb[:, :, 4:8] = 0x01
    Wb[:, :, 8:12] = 0x00
    Wb[:, :, 12:16] = 0x01
    q = np.array([[v for b in range(K // 256) for v in exact_ref.quants(Wb[n, b, 16:].tobytes())]
                  for n in range(N)], dtype=np.float64)
    ref = x.astype(np.float64) @ q.T
    y, a = oracle.qmm(x, Wb.reshape(N, -1), N, K)
    assert np.all(np.abs(y - ref) <= (K + 2) * ULP_BOUND * a)


def test_row_invariance_bitwise():
    N, K, M = 9, 1024, 5
    x = synth.acts(M, K, tensor=13, seed=15)
    W = synth.weights(N, K, tensor=14, seed=15)
    y, a = oracle.qmm(x, W, N, K)
    for m in range(M):
        y1, a1 = oracle.qmm(x[m:m + 1], W, N, K)
        assert np.array_equal(y1[0], y[m]) and np.array_equal(a1[0], a[m])


def test_row_permutation_permutes_output():
    N, K, M = 11, 512, 2
    x = synth.acts(M, K, tensor=15, seed=16)
    W = synth.weights(N, K, tensor=16, seed=16)
    perm = np.random.default_rng(0).permutation(N)
    y, _ = oracle.qmm(x, W, N, K)
    yp, _ = oracle.qmm(x, np.ascontiguousarray(W[perm]), N, K)
    assert np.array_equal(yp, y[:, perm])


def test_block_permutation_with_x_is_invariant():
    N, K, M = 5, 1280, 2
    nb = K // 256
    x = synth.acts(M, K, tensor=17, seed=17)
    W = synth.weights(N, K, tensor=18, seed=17)
    perm = np.random.default_rng(1).permutation(nb)
    Wp = W.reshape(N, nb, 144)[:, perm].reshape(N, -1).copy()
    xp = x.reshape(M, nb, 256)[:, perm].reshape(M, K).copy()
    y, a = oracle.qmm(x, W, N, K)
    yp, _ = oracle.qmm(xp, Wp, N, K)
    assert np.all(np.abs(yp - y) <= 2 * (K + 2) * ULP_BOUND * a)


def test_linearity_in_x():
    N, K = 6, 512
    W = synth.weights(N, K, tensor=19, seed=18)
    x1 = synth.acts(1, K, tensor=20, seed=18)
    x2 = synth.acts(1, K, tensor=21, seed=18)
    xs = np.concatenate([x1, x2, x1 + x2, 2.0 * x1]).astype(np.float32)
    y, a = oracle.qmm(xs, W, N, K)
    tol = 4 * (K + 2) * ULP_BOUND * (a[0] + a[1]) + 1e-300
    # x1 + x2 is rounded to fp32, so compare against the oracle's own row, not y0 + y1 exactly
    assert np.all(np.abs(y[3] - 2 * y[0]) == 0)  # doubling is exact in binary
    assert np.all(np.abs(y[2] - (y[0] + y[1])) <= tol + 2.0 ** -24 * (a[0] + a[1]))


def test_sampled_rows_match_full():
    N, K, M = 40, 512, 3
    x = synth.acts(M, K, tensor=22, seed=19)
    W = synth.weights(N, K, tensor=23, seed=19)
    y, a = oracle.qmm(x, W, N, K)
    rows = np.array([39, 0, 17, 17, 5])
    ys, as_ = oracle.qmm_rows(x, W, N, K, rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(as_, a[:, rows])


def test_thread_count_does_not_change_result():
    N, K, M = 64, 512, 2
    x = synth.acts(M, K, tensor=24, seed=20)
    W = synth.weights(N, K, tensor=25, seed=20)
    y1, a1 = oracle.qmm(x, W, N, K, nthreads=1)
    y4, a4 = oracle.qmm(x, W, N, K, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(a1, a4)


def test_rejects_bad_shapes():
    W = synth.weights(2, 512, tensor=1)
    with pytest.raises(ValueError):
        oracle.qmm(np.zeros((1, 300), np.float32), W, 2, 300)
    with pytest.raises(ValueError):
        oracle.qmm_rows(np.zeros((1, 512), np.float32), W, 2, 512, [2])


@pytest.mark.parametrize("N,K,rows", [
    (5, 512, [4, 0, 2, 2, 4, 1]),        # out of order, repeated, last row
    (3, 768, [2, 2, 1, 0]),
    (7, 256, [6, 3, 6, 0, 5, 1, 2, 4]),
])
def test_dequant_rows_match_exact_decoder(N, K, rows):
    # the read-out reference of the GPU one-hot probes: each requested row,
    # in the requested order, equals the exact rational decode of that row of
    # the packed matrix (an independent decoder); a wrong row or block offset
    # would pick up another row's bytes
    W = synth.weights(N, K, tensor=321 + N, seed=20261202)
    exact = exact_ref.matrix_weights(W.reshape(-1), N, K)
    got = oracle.dequant_rows(W, N, K, np.array(rows))
    assert got.shape == (len(rows), K)
    for i, r in enumerate(rows):
        assert [Fraction(v) for v in got[i]] == exact[r], (r, i)
    # distinct rows really differ, so the check above can tell rows apart
    assert not np.array_equal(got[0], oracle.dequant_rows(W, N, K, np.array([rows[0] - 1]))[0])


def test_dequant_rows_rejects_bad_rows():
    W = synth.weights(4, 256, tensor=9, seed=20261202)
    for bad in ([4], [-1]):
        with pytest.raises(ValueError):
            oracle.dequant_rows(W, 4, 256, np.array(bad))

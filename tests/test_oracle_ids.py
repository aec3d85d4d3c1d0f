"""Pins of the oracle's expert-indexed product (oracle.qmm_ids).

Reading of the op (the pages name MUL_MAT_ID only as a case of the op test,
"sixi-asi 0.9", section "The patch"): row m multiplies expert ids[m] of E
matrices stored back to back; rows whose id is out of range are not written.
Pinned against the independent exact evaluator, against the plain product
(one expert), and by permuting experts and ids together.
"""
from fractions import Fraction

import numpy as np
import pytest

import exact_ref
import oracle
import synth

ULP_BOUND = 2.0 ** -52


def experts(E, N, K, base):
    return np.concatenate([synth.weights(N, K, tensor=base + e).reshape(-1) for e in range(E)])


def test_ids_match_exact_row_by_row():
    E, N, K, M = 3, 3, 256, 5
    W = experts(E, N, K, 700)
    x = synth.acts(M, K, tensor=710)
    ids = np.array([2, 0, 2, -1, 1])
    y, a, written = oracle.qmm_ids(x, W, ids, E, N, K)
    mb = N * (K // 256) * 144
    assert list(written) == [True, True, True, False, True]
    assert np.all(np.isnan(y[3])) and np.all(np.isnan(a[3]))
    for m in (0, 1, 2, 4):
        e = int(ids[m])
        ye, ae = exact_ref.product(x[m:m + 1], W[e * mb:(e + 1) * mb], N, K)
        for n in range(N):
            bound = (K + 2) * ULP_BOUND * float(ae[0][n])
            assert abs(Fraction(y[m, n]) - ye[0][n]) <= Fraction(bound), (m, n)


def test_one_expert_reduces_to_the_plain_product():
    E, N, K, M = 4, 37, 512, 6
    W = experts(E, N, K, 720)
    x = synth.acts(M, K, tensor=730)
    mb = N * (K // 256) * 144
    for e in range(E):
        y, a, written = oracle.qmm_ids(x, W, np.full(M, e), E, N, K)
        y0, a0 = oracle.qmm(x, W[e * mb:(e + 1) * mb], N, K)
        assert written.all()
        assert np.array_equal(y, y0) and np.array_equal(a, a0)


def test_permuting_experts_with_ids_is_invariant():
    E, N, K, M = 5, 21, 256, 8
    W = experts(E, N, K, 740)
    x = synth.acts(M, K, tensor=750)
    ids = np.array([4, 1, 1, 3, 0, 4, 2, 1])
    y, a, _ = oracle.qmm_ids(x, W, ids, E, N, K)
    perm = np.array([3, 0, 4, 1, 2])  # new expert p holds old expert perm[p]
    mb = N * (K // 256) * 144
    Wp = np.concatenate([W[int(o) * mb:(int(o) + 1) * mb] for o in perm])
    inv = np.argsort(perm)
    yp, ap, _ = oracle.qmm_ids(x, Wp, inv[ids], E, N, K)
    assert np.array_equal(y, yp) and np.array_equal(a, ap)


def test_ids_rejects_bad_shapes():
    W = experts(2, 4, 256, 760)
    x = synth.acts(3, 256, tensor=761)
    with pytest.raises(ValueError):
        oracle.qmm_ids(x, W, np.zeros(2), 2, 4, 256)       # ids length
    with pytest.raises(ValueError):
        oracle.qmm_ids(x, W[:-1], np.zeros(3), 2, 4, 256)  # bytes

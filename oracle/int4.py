"""ORACLE -- test infrastructure only (see oracle/__init__.py for who may use it).

Plain 4-bit integer weights with one scale per 128 columns, and the skinny
product over them, in binary64, written from the format's definition; no code
is shared with the HIP library.

The pages name this layout as the plain alternative to the k-quant files (the
"sixi-asi 0.11" page, section "What did not work": 4-bit integers, one scale
per 128 columns) without fixing its bits. The plainest reading, used here:

- element: a 4-bit two's-complement integer q in [-8, 7] (symmetric, no zero
  point);
- scale: one IEEE binary16 value per 128 consecutive elements of a row along K;
- weight = scale * q.

Usual storage, which these functions take: codes uint8 [N, K/2] with element
2i of a row in the low nibble of byte i and 2i+1 in the high nibble; scales
uint16 [N, K/128], binary16 bit patterns, scale j covering elements
128j .. 128j+127.

Pins (tests/test_oracle_int4.py): the two's-complement table and hand-decoded
binary16 values (tests/golden/int4.txt); every binary16 pattern against
numpy's float16 conversion; one-hot code and scale probes that fix each
position; brute-force sums; zero codes giving exact zeros.
"""
import numpy as np


def int4_value(code):
    """Value of a 4-bit two's-complement code (bit 3 is the sign)."""
    code = int(code) & 0xF
    return code - 16 if code >= 8 else code


def f16_value(bits):
    """Value of an IEEE binary16 bit pattern: 1 sign bit, 5 exponent bits with
    bias 15, 10 fraction bits; exponent 0 is subnormal (2^-14 x 0.f), 31 is
    infinity (fraction 0) or NaN."""
    bits = int(bits) & 0xFFFF
    s, e, f = bits >> 15, (bits >> 10) & 31, bits & 1023
    if e == 31:
        mag = float("inf") if f == 0 else float("nan")
    elif e == 0:
        mag = 2.0 ** -14 * (f / 1024.0)
    else:
        mag = 2.0 ** (e - 15) * (1.0 + f / 1024.0)
    return -mag if s else mag


_INT4 = np.array([int4_value(c) for c in range(16)], dtype=np.float64)
_F16 = None


def _f16_table():
    global _F16
    if _F16 is None:
        _F16 = np.array([f16_value(b) for b in range(65536)], dtype=np.float64)
    return _F16


def _check(codes, scales, K):
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    if codes.dtype != np.uint8 or scales.dtype != np.uint16:
        raise TypeError("codes must be uint8, scales uint16 binary16 patterns")
    if K <= 0 or K % 128:
        raise ValueError("K must be a positive multiple of 128")
    if codes.ndim != 2 or codes.shape[1] != K // 2:
        raise ValueError("codes must be [N, K/2]")
    if scales.ndim != 2 or scales.shape != (codes.shape[0], K // 128):
        raise ValueError("scales must be [N, K/128]")
    return codes, scales


def dequant_rows(codes, scales, K, rows=None):
    """fp64 weights [len(rows), K] of the given rows (all rows when None)."""
    codes, scales = _check(codes, scales, K)
    if rows is None:
        rows = np.arange(codes.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    c = codes[rows]
    q = np.empty((len(rows), K), dtype=np.uint8)
    q[:, 0::2] = c & 0xF   # element 2i: low nibble of byte i
    q[:, 1::2] = c >> 4    # element 2i+1: high nibble
    w = _INT4[q]
    w *= np.repeat(_f16_table()[scales[rows]], 128, axis=1)  # scale j: elements 128j..128j+127
    return w


def qmm_int4(x, codes, scales, N, K, rows=None, chunk=2048):
    """y[m, n] = sum_k x[m, k] * w[n, k] in fp64 for n in rows (all when None),
    with a[m, n] = sum_k |x[m, k] * w[n, k]| (the scale of the error gate).
    x: fp32 or fp64 [M, K]. Returns (y, a), each [M, len(rows)]."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M, K]")
    if codes.shape[0] != N:
        raise ValueError("codes must have N rows")
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows, dtype=np.int64)
    y = np.empty((x.shape[0], len(rows)))
    a = np.empty_like(y)
    ax = np.abs(x)
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        w = dequant_rows(codes, scales, K, r)
        y[:, c0:c0 + len(r)] = x @ w.T
        a[:, c0:c0 + len(r)] = ax @ np.abs(w).T
    return y, a

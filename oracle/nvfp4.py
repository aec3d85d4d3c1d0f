"""ORACLE -- test infrastructure only (see oracle/__init__.py for who may use it).

Block-scaled FP4 weights ("NVFP4") and the skinny product over them, in
binary64, written from the format definitions; no code is shared with the HIP
library.

The pages name the format and measure a W4A16 product over it (FlashRT issue
#153: the NVFP4 W4A16 GEMM, its per-shape tile bench for lm_head and gate+up
at 1 and 7 rows); they do not define its bits. Those come from public specs:

- element: FP4 E2M1 of the OCP Microscaling Formats (MX) specification v1.0:
  1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, no infinity or NaN;
  exponent field 0 is subnormal (0.m x 2^0), otherwise 2^(e-1) x 1.m;
- block scale: FP8 E4M3 of the OCP 8-bit floating point specification (OFP8):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinity, the
  codes S.1111.111 are NaN; exponent field 0 is subnormal (2^-6 x 0.mmm);
- NVFP4: one E4M3 scale per 16 consecutive elements of a row and one fp32
  scale per tensor; weight = tensor_scale * scale * element.

Usual storage, which these functions take: elems uint8 [N, K/2] with element
2i of a row in the low nibble of byte i and 2i+1 in the high nibble; scales
uint8 [N, K/16], scale j covering elements 16j .. 16j+15.

Pins (tests/test_oracle_nvfp4.py): the spec's E2M1 value table
(tests/golden/nvfp4.txt); every E4M3 code against torch's float8_e4m3fn
conversion and the spec's named values; one-hot element and scale probes that
fix each code's position; brute-force sums; linearity in the tensor scale.
"""
import numpy as np


def e2m1_value(code):
    """Value of a 4-bit E2M1 code (sign bit 3, exponent bits 2..1, mantissa bit 0)."""
    code = int(code) & 0xF
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def e4m3_value(code):
    """Value of an 8-bit E4M3 code (sign bit 7, exponent bits 6..3, mantissa 2..0)."""
    code = int(code) & 0xFF
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = 2.0 ** -6 * (m / 8.0) if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


_E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def _check(elems, scales, K):
    elems = np.ascontiguousarray(elems)
    scales = np.ascontiguousarray(scales)
    if elems.dtype != np.uint8 or scales.dtype != np.uint8:
        raise TypeError("elems and scales must be uint8 codes")
    if K <= 0 or K % 16:
        raise ValueError("K must be a positive multiple of 16")
    if elems.ndim != 2 or elems.shape[1] != K // 2:
        raise ValueError("elems must be [N, K/2]")
    if scales.ndim != 2 or scales.shape != (elems.shape[0], K // 16):
        raise ValueError("scales must be [N, K/16]")
    return elems, scales


def dequant_rows(elems, scales, tensor_scale, K, rows=None):
    """fp64 weights [len(rows), K] of the given rows (all rows when None)."""
    elems, scales = _check(elems, scales, K)
    if rows is None:
        rows = np.arange(elems.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    e = elems[rows]
    codes = np.empty((len(rows), K), dtype=np.uint8)
    codes[:, 0::2] = e & 0xF   # element 2i: low nibble of byte i
    codes[:, 1::2] = e >> 4    # element 2i+1: high nibble
    w = _E2M1[codes]
    w *= np.repeat(_E4M3[scales[rows]], 16, axis=1)  # scale j covers elements 16j..16j+15
    w *= float(tensor_scale)
    return w


def qmm_nvfp4(x, elems, scales, tensor_scale, N, K, rows=None, chunk=2048):
    """y[m, n] = sum_k x[m, k] * w[n, k] in fp64 for n in rows (all when None),
    with a[m, n] = sum_k |x[m, k] * w[n, k]| (the scale of the error gate).
    x: fp32 or fp64 [M, K]. Returns (y, a), each [M, len(rows)]."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M, K]")
    if elems.shape[0] != N:
        raise ValueError("elems must have N rows")
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows, dtype=np.int64)
    y = np.empty((x.shape[0], len(rows)))
    a = np.empty_like(y)
    ax = np.abs(x)
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        w = dequant_rows(elems, scales, tensor_scale, K, r)
        y[:, c0:c0 + len(r)] = x @ w.T
        a[:, c0:c0 + len(r)] = ax @ np.abs(w).T
    return y, a

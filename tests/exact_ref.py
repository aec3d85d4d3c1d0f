"""An exact-rational evaluator of the skinny quantized product, for tiny shapes.

Independent of the oracle: its own binary16 decoder, its own unpacking of the
12 scale bytes (by absolute bit positions inside the 96-bit little-endian
field) and of the quants (walking the bytes and scattering both nibbles),
all in fractions.Fraction, so products and sums are exact.

Format reading (the same one the oracle states; the pages name the Q4_K k-quant
of "sixi-asi 0.9", section "Numbers", but print no byte map).
"""
from fractions import Fraction


def f16_exact(bits):
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 31
    f = bits & 1023
    if e == 31:
        raise ValueError("inf/nan has no exact value")
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * Fraction(1024 + f, 1 << 10) * (Fraction(2) ** (e - 15))


def _bits(field, lo, width):
    return (field >> lo) & ((1 << width) - 1)


def scales_mins(s12):
    """[(sc_j, m_j)] for j = 0..7 from the 12 packed bytes, by bit position."""
    field = int.from_bytes(bytes(s12), "little")  # byte t occupies bits 8t..8t+7
    out = []
    for j in range(8):
        if j < 4:
            sc = _bits(field, 8 * j, 6)
            mn = _bits(field, 8 * (j + 4), 6)
        else:
            t = j - 4
            sc = _bits(field, 8 * (8 + t), 4) + 16 * _bits(field, 8 * t + 6, 2)
            mn = _bits(field, 8 * (8 + t) + 4, 4) + 16 * _bits(field, 8 * (4 + t) + 6, 2)
        out.append((sc, mn))
    return out


def quants(qs128):
    q = [None] * 256
    for idx, byte in enumerate(qs128):
        group, lane = divmod(idx, 32)
        q[64 * group + lane] = byte & 15
        q[64 * group + 32 + lane] = byte >> 4
    return q


def block_weights(blk):
    blk = bytes(blk)
    d = f16_exact(blk[0] | (blk[1] << 8))
    dmin = f16_exact(blk[2] | (blk[3] << 8))
    sm = scales_mins(blk[4:16])
    q = quants(blk[16:144])
    return [d * sm[i // 32][0] * q[i] - dmin * sm[i // 32][1] for i in range(256)]


def matrix_weights(W, N, K):
    W = bytes(W)
    nb = K // 256
    rows = []
    for n in range(N):
        row = []
        for b in range(nb):
            off = (n * nb + b) * 144
            row.extend(block_weights(W[off:off + 144]))
        rows.append(row)
    return rows


def product(x, W, N, K):
    """(y, a) exact: y[m][n] = sum_k x[m][k] w[n][k], a[m][n] = sum_k |x w|."""
    w = matrix_weights(W, N, K)
    xs = [[Fraction(float(v)) for v in row] for row in x]
    y = [[sum(xr[k] * w[n][k] for k in range(K)) for n in range(N)] for xr in xs]
    a = [[sum(abs(xr[k] * w[n][k]) for k in range(K)) for n in range(N)] for xr in xs]
    return y, a

"""ORACLE -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. It is a plain binary64 CPU implementation of the skinny quantized
product written from its definition (qk_oracle.c cites the passages); it shares
no code with the HIP library and imports nothing from it.

Pins: see qk_oracle.c. GGUF file compatibility of the byte layout is parity
unpinned (no GGUF file is available to compare against).

oracle.nvfp4 is the oracle of the block-scaled FP4 product (numpy, binary64;
its header gives the format's sources and pins).
oracle.int4 is the oracle of the plain 4-bit integer product, one binary16
scale per 128 columns (numpy, binary64; its header gives the reading and pins).
oracle.gdn is the oracle of the Gated DeltaNet recurrent update with the
replay of a row log (numpy, binary64; parity unpinned against the pages, which
give the update's inputs but not its equation; its header gives the source and
the pins).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qk_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIBRARY names another build of qk_oracle.c to load instead (the
# sanitizer build of the tests)
_LOAD = os.environ.get("ORACLE_LIBRARY") or _LIB


def build():
    """Compile qk_oracle.c into liboracle.so: gcc -O2, no -ffast-math, no SIMD intrinsics."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LOAD == _LIB and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LOAD)
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_scale_min.argtypes = [ctypes.c_void_p, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        lib.oracle_scale_min.restype = None
        lib.oracle_dequant_block.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_dequant_block.restype = None
        lib.oracle_dequant_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_dequant_rows.restype = ctypes.c_int
        lib.oracle_qmm_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int]
        lib.oracle_qmm_rows.restype = ctypes.c_int
        lib.oracle_qmm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int]
        lib.oracle_qmm.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _u8(W):
    W = np.ascontiguousarray(W)
    if W.dtype != np.uint8:
        raise TypeError("W must be uint8 bytes")
    return W


def f16_to_f64(bits):
    return float(_load().oracle_f16_to_f64(int(bits) & 0xFFFF))


def scale_min(block, j):
    """(sc_j, m_j) of a 144-byte block."""
    b = _u8(np.frombuffer(bytes(block), dtype=np.uint8) if isinstance(block, (bytes, bytearray)) else block)
    sc, m = ctypes.c_int(), ctypes.c_int()
    _load().oracle_scale_min(b.ctypes.data + 4, int(j), ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def dequant_block(block):
    """The 256 binary64 weights of one 144-byte block."""
    b = _u8(np.frombuffer(bytes(block), dtype=np.uint8) if isinstance(block, (bytes, bytearray)) else block)
    if b.size != 144:
        raise ValueError("a block is 144 bytes")
    w = np.empty(256, dtype=np.float64)
    _load().oracle_dequant_block(b.ctypes.data, w.ctypes.data)
    return w


def dequant_rows(W, N, K, rows):
    """Dequantized rows [len(rows), K] of the packed N x K matrix W."""
    W = _u8(W)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, int(K)), dtype=np.float64)
    if W.size != N * (K // 256) * 144:
        raise ValueError("W size does not match N, K")
    rc = _load().oracle_dequant_rows(W.ctypes.data, int(N), int(K), rows.ctypes.data,
                                     rows.size, out.ctypes.data)
    if rc:
        raise ValueError("oracle_dequant_rows: bad arguments")
    return out


def qmm_rows(x, W, N, K, rows, nthreads=0):
    """(y, a) for the selected rows: y[m][r] = sum_k x[m,k] w[rows[r],k], a = sum_k |x w|."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    W = _u8(W)
    M = x.shape[0]
    if x.shape[1] != K or W.size != N * (K // 256) * 144:
        raise ValueError("shape mismatch")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((M, rows.size), dtype=np.float64)
    a = np.empty((M, rows.size), dtype=np.float64)
    rc = _load().oracle_qmm_rows(x.ctypes.data, W.ctypes.data, M, int(N), int(K),
                                 rows.ctypes.data, rows.size, y.ctypes.data, a.ctypes.data,
                                 int(nthreads))
    if rc:
        raise ValueError("oracle_qmm_rows failed (%d)" % rc)
    return y, a


def qmm(x, W, N, K, nthreads=0):
    """(y, a): y[M,N] = x . dequant(W)^T in binary64 and a = sum_k |x w| (the tolerance scale)."""
    return qmm_rows(x, W, N, K, np.arange(int(N), dtype=np.int64), nthreads)


def threads():
    return int(_load().oracle_threads())


def qmm_ids(x, W_experts, ids, E, N, K, nthreads=0):
    """Expert-indexed product: y[m] = x[m] . dequant(W_experts[ids[m]])^T, in binary64.

    W_experts holds E packed N x K matrices back to back. Returns (y, a, written):
    rows whose id lies outside [0, E) are not written (y and a are NaN there and
    written[m] is False). This is the definition row group by row group: each
    distinct expert's rows go through qmm_rows with that expert's matrix.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    W_experts = _u8(W_experts)
    ids = np.asarray(ids, dtype=np.int64)
    M = x.shape[0]
    mb = int(N) * (int(K) // 256) * 144
    if W_experts.size != int(E) * mb or ids.shape != (M,):
        raise ValueError("shape mismatch")
    y = np.full((M, int(N)), np.nan)
    a = np.full((M, int(N)), np.nan)
    written = (ids >= 0) & (ids < int(E))
    for e in sorted(set(int(v) for v in ids[written])):
        rows = np.nonzero(ids == e)[0]
        ye, ae = qmm(x[rows], W_experts[e * mb:(e + 1) * mb], N, K, nthreads)
        y[rows] = ye
        a[rows] = ae
    return y, a, written

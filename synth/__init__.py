"""Seeded synthetic inputs (weights as packed super-blocks, fp32 activations).

This module is the one input source that both the oracle side and the HIP side
use. It holds none of the product's arithmetic: bytes 4..143 of every 144-byte
super-block are uniform random bytes, so each 6-bit scale, 6-bit min and 4-bit
quant inside them is uniform over its range whatever the packing; bytes 0..3
are the binary16 values d and dmin = f16(|z|*1e-2). Activations are
f32(scale*z), z ~ N(0,1). The streams are counter-based SplitMix64 (Steele, Lea
and Flood, OOPSLA 2014) keyed by (seed, tensor id, field), so every value is a
pure function of its index and the output does not depend on the thread count.

Workload: synthetic stand-ins for the Q4_K_M GGUF weights and the activations
of the 27B model on "sixi-asi 0.9" (section "Numbers"); no trained weights are
used.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

DEFAULT_SEED = 20261202
BLOCK_BYTES = 144
BLOCK_WEIGHTS = 256
FIELD_BYTES, FIELD_D, FIELD_DMIN, FIELD_X, FIELD_FP4_ELEMS, FIELD_FP4_SCALES = 1, 2, 3, 4, 5, 6
# streams of the recurrent-update inputs
(FIELD_GDN_STATE, FIELD_GDN_Q, FIELD_GDN_K, FIELD_GDN_V, FIELD_GDN_GATE,
 FIELD_GDN_BETA) = 16, 17, 18, 19, 20, 21


def build():
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.synth_weights.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_void_p]
        lib.synth_weights.restype = ctypes.c_int
        lib.synth_acts.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        lib.synth_acts.restype = ctypes.c_int
        lib.synth_nvfp4.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_nvfp4.restype = ctypes.c_int
        lib.synth_int4.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_int4.restype = ctypes.c_int
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        lib.synth_normal_f32.restype = ctypes.c_int
        lib.synth_uniform_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_void_p]
        lib.synth_uniform_f32.restype = ctypes.c_int
        lib.synth_f64_to_f16.argtypes = [ctypes.c_double]
        lib.synth_f64_to_f16.restype = ctypes.c_uint16
        lib.synth_word.argtypes = [ctypes.c_uint64] * 4
        lib.synth_word.restype = ctypes.c_uint64
        lib.synth_normal.argtypes = [ctypes.c_uint64] * 4
        lib.synth_normal.restype = ctypes.c_double
        lib.synth_threads.argtypes = []
        lib.synth_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def weight_bytes(n_rows, K):
    return int(n_rows) * (int(K) // BLOCK_WEIGHTS) * BLOCK_BYTES


def weights(n_rows, K, tensor, seed=DEFAULT_SEED, out=None):
    """Packed super-blocks for an n_rows x K matrix: uint8 array [n_rows, K/256*144]."""
    if K <= 0 or K % BLOCK_WEIGHTS:
        raise ValueError("K must be a positive multiple of 256")
    shape = (int(n_rows), int(K) // BLOCK_WEIGHTS * BLOCK_BYTES)
    if out is None:
        out = np.empty(shape, dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous and out.size == shape[0] * shape[1]
    rc = _load().synth_weights(seed, tensor, int(n_rows), int(K), out.ctypes.data)
    if rc:
        raise RuntimeError("synth_weights failed")
    return out


def acts(M, K, tensor, seed=DEFAULT_SEED, scale=1.0, out=None):
    """fp32 activations [M, K], x = f32(scale * z), z ~ N(0,1)."""
    if out is None:
        out = np.empty((int(M), int(K)), dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == M * K
    rc = _load().synth_acts(seed, tensor, int(M), int(K), float(scale), out.ctypes.data)
    if rc:
        raise RuntimeError("synth_acts failed")
    return out


def nvfp4(n_rows, K, tensor, seed=DEFAULT_SEED):
    """Block-scaled FP4 weights in the usual two-array layout: (elems uint8
    [n_rows, K/2], two 4-bit codes per byte, element 2i in the low nibble;
    scales uint8 [n_rows, K/16], one 8-bit scale code per 16 elements).
    Random bit fields only; see synth_nvfp4 in synth.c."""
    if K <= 0 or K % 16:
        raise ValueError("K must be a positive multiple of 16")
    elems = np.empty((int(n_rows), int(K) // 2), dtype=np.uint8)
    scales = np.empty((int(n_rows), int(K) // 16), dtype=np.uint8)
    rc = _load().synth_nvfp4(seed, tensor, int(n_rows), int(K), elems.ctypes.data,
                             scales.ctypes.data)
    if rc:
        raise RuntimeError("synth_nvfp4 failed")
    return elems, scales


def int4(n_rows, K, tensor, seed=DEFAULT_SEED):
    """Plain 4-bit integer weights in the usual two-array layout: (codes uint8
    [n_rows, K/2], two 4-bit two's-complement codes per byte, element 2i in
    the low nibble; scales uint16 [n_rows, K/128], binary16 bit patterns, one
    per 128 elements). Random fields only; see synth_int4 in synth.c."""
    if K <= 0 or K % 128:
        raise ValueError("K must be a positive multiple of 128")
    codes = np.empty((int(n_rows), int(K) // 2), dtype=np.uint8)
    scales = np.empty((int(n_rows), int(K) // 128), dtype=np.uint16)
    rc = _load().synth_int4(seed, tensor, int(n_rows), int(K), codes.ctypes.data,
                            scales.ctypes.data)
    if rc:
        raise RuntimeError("synth_int4 failed")
    return codes, scales


def normal_f32(n, tensor, field, seed=DEFAULT_SEED, scale=1.0):
    """fp32 [n], f32(scale * z), z ~ N(0,1), of stream (seed, tensor, field)."""
    out = np.empty(int(n), dtype=np.float32)
    if _load().synth_normal_f32(seed, tensor, field, int(n), float(scale), out.ctypes.data):
        raise RuntimeError("synth_normal_f32 failed")
    return out


def uniform_f32(n, tensor, field, lo, hi, seed=DEFAULT_SEED):
    """fp32 [n], f32(lo + (hi - lo) * w), w uniform in [0, 1) (53 bits)."""
    out = np.empty(int(n), dtype=np.float32)
    if _load().synth_uniform_f32(seed, tensor, field, int(n), float(lo), float(hi), out.ctypes.data):
        raise RuntimeError("synth_uniform_f32 failed")
    return out


def _unit_rows(a, scale=1.0):
    # rows of a rescaled to Euclidean norm `scale` (binary64), rounded to fp32
    a64 = a.astype(np.float64)
    n = np.sqrt((a64 * a64).sum(axis=-1, keepdims=True))
    return (scale * a64 / np.where(n > 0, n, 1.0)).astype(np.float32)


def gdn_rows(B, R, H, dk, dv, tensor, seed=DEFAULT_SEED, queries=True):
    """Per-row inputs of the recurrent update for B sequences of R rows and H
    heads: dict of q [B,R,H,dk] (unit norm times dk^-1/2; omitted when
    queries is False), k [B,R,H,dk] (unit norm), v [B,R,H,dv] ~ N(0,1),
    gate [B,R,H] uniform in [0.85, 1), beta [B,R,H] uniform in [0.05, 0.95).
    The shapes and distributions of a Gated DeltaNet layer's inputs after its
    key/query normalization; no trained weights."""
    out = {}
    shape = (B, R, H)
    n = B * R * H
    if queries:
        out["q"] = _unit_rows(normal_f32(n * dk, tensor, FIELD_GDN_Q, seed).reshape(shape + (dk,)),
                              dk ** -0.5)
    out["k"] = _unit_rows(normal_f32(n * dk, tensor, FIELD_GDN_K, seed).reshape(shape + (dk,)))
    out["v"] = normal_f32(n * dv, tensor, FIELD_GDN_V, seed).reshape(shape + (dv,))
    out["gate"] = uniform_f32(n, tensor, FIELD_GDN_GATE, 0.85, 1.0, seed).reshape(shape)
    out["beta"] = uniform_f32(n, tensor, FIELD_GDN_BETA, 0.05, 0.95, seed).reshape(shape)
    return out


def gdn_state(B, H, dk, dv, tensor, seed=DEFAULT_SEED, scale=0.05):
    """Base states [B,H,dk,dv] fp32, f32(scale * z): the layout keeps the key
    index outer and the value index inner (element [b,h,e,i] is row i, column
    e of the head's value-by-key state matrix)."""
    return normal_f32(B * H * dk * dv, tensor, FIELD_GDN_STATE, seed, scale).reshape(B, H, dk, dv)


def f64_to_f16_bits(v):
    return int(_load().synth_f64_to_f16(float(v)))


def word(seed, tensor, field, i):
    return int(_load().synth_word(seed, tensor, field, i))


def normal(seed, tensor, field, i):
    return float(_load().synth_normal(seed, tensor, field, i))


def threads():
    return int(_load().synth_threads())

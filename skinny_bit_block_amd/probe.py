"""Binding of the measurement probes (include/qmm_probe.h) in libqmm.so:
argument marshalling only."""
import ctypes

from . import load as _load_lib, _check

EXPORTS = ["qmm_probe_read", "qmm_probe_empty", "qmm_probe_clock"]

_done = False


def _lib():
    global _done
    lib = _load_lib()
    if not _done:
        vp = ctypes.c_void_p
        lib.qmm_probe_read.argtypes = [vp, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, vp, vp]
        lib.qmm_probe_read.restype = ctypes.c_int
        lib.qmm_probe_empty.argtypes = [ctypes.c_int, vp]
        lib.qmm_probe_empty.restype = ctypes.c_int
        lib.qmm_probe_clock.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int), vp]
        lib.qmm_probe_clock.restype = ctypes.c_int
        _done = True
    return lib


def qmm_probe_read(buf_ptr, nbytes, grid, block, sink_ptr, stream_ptr):
    return _check(_lib().qmm_probe_read(buf_ptr, int(nbytes), int(grid), int(block), sink_ptr,
                                        stream_ptr))


def qmm_probe_empty(grid, stream_ptr):
    return _check(_lib().qmm_probe_empty(int(grid), stream_ptr))


def qmm_probe_clock(counts_ptr, grid, iters, stream_ptr):
    """Launch the clock probe; returns the constant counter's rate in kHz."""
    khz = ctypes.c_int(0)
    _check(_lib().qmm_probe_clock(counts_ptr, int(grid), int(iters), ctypes.byref(khz), stream_ptr))
    return khz.value

"""Raw HIP events for the library's launch-event hook (qmm_set_launch_events).

The HIP runtime that torch loaded is the one the library uses (one soname), so
events made here, the library's launches and torch's streams all belong to the
same runtime. A torch.cuda.Event has no HIP event until torch records it, and
torch does not see a record made by the library, so the hook takes these.
"""
import ctypes

_rt = None


def _runtime():
    global _rt
    if _rt is None:
        _rt = ctypes.CDLL("libamdhip64.so.7")
        _rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    return _rt


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed: hipError %d" % (what, rc))


class EventPool:
    """Pairs of HIP events, made once and reused; elapsed() reads a pair in ms."""

    def __init__(self, pairs):
        rt = _runtime()
        self.pairs = []
        for _ in range(pairs):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            _check(rt.hipEventCreate(ctypes.byref(a)), "hipEventCreate")
            _check(rt.hipEventCreate(ctypes.byref(b)), "hipEventCreate")
            self.pairs.append((a.value, b.value))

    def elapsed_ms(self, i):
        rt = _runtime()
        a, b = self.pairs[i]
        _check(rt.hipEventSynchronize(b), "hipEventSynchronize")
        f = ctypes.c_float()
        _check(rt.hipEventElapsedTime(ctypes.byref(f), a, b), "hipEventElapsedTime")
        return f.value

    def close(self):
        rt = _runtime()
        for a, b in self.pairs:
            rt.hipEventDestroy(a)
            rt.hipEventDestroy(b)
        self.pairs = []

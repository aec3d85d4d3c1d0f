"""Python binding of libqmm.so: the skinny quantized product on MI355X.

    y[M,N] = x[M,K] . dequant(W)[N,K]^T,  M = 1..32,

with W in 144-byte / 256-weight Q4_K super-blocks (the C header include/qmm.h
states the format, the layouts and the error behaviour). This module only
marshals arguments: the same names as the C entry points, torch tensors in,
raw device pointers out. Every step of the product runs in the HIP kernels of
libqmm.so; there is no fallback path, and a missing library is an error.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# QMM_LIBRARY names another build of the same sources to load instead (the
# host-sanitizer build of the tests)
LIB_PATH = os.environ.get("QMM_LIBRARY") or os.path.join(HERE, "libqmm.so")

QMM_OK = 0
QMM_ERR_INVALID_ARG = -1
QMM_ERR_SHAPE = -2
QMM_ERR_ALIGN = -3
QMM_ERR_NO_DEVICE = -4
QMM_ERR_OOM = -5
QMM_ERR_HIP = -6
QMM_ERR_OVERLAP = -7
QMM_ERR_SCRATCH = -8
QMM_MAX_M = 32
QMM_DEVICE_NONE = -1  # planning-only handle: plans and checks arguments, never launches

KERNEL_AUTO, KERNEL_VECTOR, KERNEL_TILED = 0, 1, 2
FORMAT_KQUANT, FORMAT_NVFP4, FORMAT_INT4 = 0, 1, 2
KERNEL_NAMES = {KERNEL_VECTOR: "vector", KERNEL_TILED: "tiled"}

EXPORTS = ["qmm_create", "qmm_run", "qmm_run_static", "qmm_run_ids", "qmm_run_nvfp4", "qmm_nvfp4_repack",
           "qmm_run_int4", "qmm_int4_repack", "qmm_destroy", "qmm_status_string", "qmm_weight_bytes",
           "qmm_query_plan", "qmm_set_kernel", "qmm_set_shape", "qmm_set_wave_splits",
           "qmm_switch_point", "qmm_set_launch_events", "qmm_query_plan_format"]


class qmm_plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("waves_per_wg", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("grid_x", ctypes.c_int32),
                ("blocks_per_split", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("wave_splits", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def load():
    """Load libqmm.so (built by build.py / __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqmm.so is not built: run `python -m skinny_bit_block_amd.build` "
                               "or __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.qmm_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int]
        lib.qmm_create.restype = ctypes.c_int
        lib.qmm_run.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        lib.qmm_run.restype = ctypes.c_int
        lib.qmm_run_static.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        lib.qmm_run_static.restype = ctypes.c_int
        lib.qmm_run_ids.argtypes = [vp, vp, vp, vp, i64, vp, i64, i64, i64, vp]
        lib.qmm_run_ids.restype = ctypes.c_int
        lib.qmm_run_nvfp4.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i64, i64, vp]
        lib.qmm_run_nvfp4.restype = ctypes.c_int
        lib.qmm_nvfp4_repack.argtypes = [vp, vp, i64, i64, vp]
        lib.qmm_nvfp4_repack.restype = ctypes.c_int
        lib.qmm_run_int4.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        lib.qmm_run_int4.restype = ctypes.c_int
        lib.qmm_int4_repack.argtypes = [vp, vp, i64, i64, vp]
        lib.qmm_int4_repack.restype = ctypes.c_int
        lib.qmm_destroy.argtypes = [vp]
        lib.qmm_destroy.restype = ctypes.c_int
        lib.qmm_status_string.argtypes = [ctypes.c_int]
        lib.qmm_status_string.restype = ctypes.c_char_p
        lib.qmm_weight_bytes.argtypes = [i64, i64]
        lib.qmm_weight_bytes.restype = ctypes.c_uint64
        lib.qmm_query_plan.argtypes = [vp, i64, i64, i64, ctypes.POINTER(qmm_plan)]
        lib.qmm_query_plan.restype = ctypes.c_int
        lib.qmm_query_plan_format.argtypes = [vp, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                              ctypes.POINTER(qmm_plan)]
        lib.qmm_query_plan_format.restype = ctypes.c_int
        lib.qmm_set_kernel.argtypes = [vp, ctypes.c_int]
        lib.qmm_set_kernel.restype = ctypes.c_int
        lib.qmm_set_shape.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.qmm_set_shape.restype = ctypes.c_int
        lib.qmm_set_wave_splits.argtypes = [vp, ctypes.c_int]
        lib.qmm_set_wave_splits.restype = ctypes.c_int
        lib.qmm_switch_point.argtypes = [vp, i64, i64]
        lib.qmm_switch_point.restype = ctypes.c_int
        lib.qmm_set_launch_events.argtypes = [vp, vp, vp]
        lib.qmm_set_launch_events.restype = ctypes.c_int
        _lib = lib
    return _lib


class QmmError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(qmm_status_string(status))


def _check(status):
    if status != QMM_OK:
        raise QmmError(status)
    return status


def qmm_status_string(status):
    return load().qmm_status_string(int(status)).decode()


def qmm_weight_bytes(N, K):
    return int(load().qmm_weight_bytes(int(N), int(K)))


def qmm_create(device=0):
    """A handle on HIP device `device` (QMM_DEVICE_NONE: planning only)."""
    h = ctypes.c_void_p()
    _check(load().qmm_create(ctypes.byref(h), int(device)))
    return h


def qmm_destroy(h):
    return _check(load().qmm_destroy(h))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def qmm_run(h, x, W_blocks, y, M, N, K, stream=None):
    """Enqueue y = x . dequant(W_blocks)^T on `stream` (default: torch's current stream).

    x: fp32 [M,K] device tensor; W_blocks: uint8 device tensor of N*K/256*144 bytes;
    y: fp32 [M,N] device tensor (overwritten). Raw integer pointers are accepted too.
    """
    for name, t, dt in (("x", x, "float32"), ("W_blocks", W_blocks, "uint8"), ("y", y, "float32")):
        if t is not None and not isinstance(t, int):
            if not t.is_cuda:
                raise ValueError("%s must be a device tensor" % name)
            if str(t.dtype) != "torch." + dt:
                raise ValueError("%s must be %s" % (name, dt))
            if not t.is_contiguous():
                raise ValueError("%s must be contiguous" % name)
    if x is not None and not isinstance(x, int) and x.numel() < M * K:
        raise ValueError("x has fewer than M*K elements")
    if y is not None and not isinstance(y, int) and y.numel() < M * N:
        raise ValueError("y has fewer than M*N elements")
    if W_blocks is not None and not isinstance(W_blocks, int) and W_blocks.numel() < qmm_weight_bytes(N, K):
        raise ValueError("W_blocks has fewer than N*K/256*144 bytes")
    return _check(load().qmm_run(h, _ptr(x), _ptr(W_blocks), _ptr(y), int(M), int(N), int(K),
                                 _stream(stream)))


def qmm_run_static(x, W_blocks, y, M, N, K, stream=None):
    """qmm_run without a handle and without allocating: the library's static
    per-device scratch serves as split-K workspace (QMM_ERR_SCRATCH when the
    call's plan needs more). Runs on the current device; arguments as for
    qmm_run."""
    _check_group_args(x, W_blocks, y, M, N, K)
    return _check(load().qmm_run_static(_ptr(x), _ptr(W_blocks), _ptr(y), int(M), int(N), int(K),
                                        _stream(stream)))


def qmm_run_static_raw(x_ptr, w_ptr, y_ptr, M, N, K, stream_ptr):
    """The C call with raw pointers; returns the status instead of raising."""
    return int(load().qmm_run_static(x_ptr, w_ptr, y_ptr, int(M), int(N), int(K), stream_ptr))


def qmm_run_ids(h, x, W_experts, ids, E, y, M, N, K, stream=None):
    """Enqueue y[m] = x[m] . dequant(W_experts[ids[m]])^T on `stream`.

    W_experts: uint8 device tensor of E matrices of N*K/256*144 bytes each;
    ids: int32 device tensor of M expert indices (rows with an id outside [0, E)
    are not written). Other arguments as for qmm_run.
    """
    for name, t, dt in (("x", x, "float32"), ("W_experts", W_experts, "uint8"),
                        ("ids", ids, "int32"), ("y", y, "float32")):
        if t is not None and not isinstance(t, int):
            if not t.is_cuda:
                raise ValueError("%s must be a device tensor" % name)
            if str(t.dtype) != "torch." + dt:
                raise ValueError("%s must be %s" % (name, dt))
            if not t.is_contiguous():
                raise ValueError("%s must be contiguous" % name)
    if x is not None and not isinstance(x, int) and x.numel() < M * K:
        raise ValueError("x has fewer than M*K elements")
    if y is not None and not isinstance(y, int) and y.numel() < M * N:
        raise ValueError("y has fewer than M*N elements")
    if ids is not None and not isinstance(ids, int) and ids.numel() < M:
        raise ValueError("ids has fewer than M elements")
    if W_experts is not None and not isinstance(W_experts, int) and \
            W_experts.numel() < qmm_weight_bytes(N, K) * E:
        raise ValueError("W_experts has fewer than E*N*K/256*144 bytes")
    return _check(load().qmm_run_ids(h, _ptr(x), _ptr(W_experts), _ptr(ids), int(E), _ptr(y),
                                     int(M), int(N), int(K), _stream(stream)))


def qmm_nvfp4_repack(elems, scales, N, K):
    """Block-scaled FP4 weights from the usual layout (numpy uint8 elems [N, K/2],
    element 2i in the low nibble of byte i; scales [N, K/16]) to the library's
    groups: a numpy uint8 array [N, K/256*144] (host memory; copy it to the
    device for qmm_run_nvfp4)."""
    import numpy as np
    elems = np.ascontiguousarray(elems, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if elems.size != N * K // 2 or scales.size != N * K // 16:
        raise ValueError("elems must hold N*K/2 bytes and scales N*K/16")
    out = np.empty((int(N), int(K) // 256 * 144), dtype=np.uint8)
    _check(load().qmm_nvfp4_repack(elems.ctypes.data, scales.ctypes.data, int(N), int(K),
                                   out.ctypes.data))
    return out


def _check_group_args(x, W_groups, y, M, N, K):
    for name, t, dt in (("x", x, "float32"), ("W_groups", W_groups, "uint8"), ("y", y, "float32")):
        if t is not None and not isinstance(t, int):
            if not t.is_cuda:
                raise ValueError("%s must be a device tensor" % name)
            if str(t.dtype) != "torch." + dt:
                raise ValueError("%s must be %s" % (name, dt))
            if not t.is_contiguous():
                raise ValueError("%s must be contiguous" % name)
    if x is not None and not isinstance(x, int) and x.numel() < M * K:
        raise ValueError("x has fewer than M*K elements")
    if y is not None and not isinstance(y, int) and y.numel() < M * N:
        raise ValueError("y has fewer than M*N elements")
    if W_groups is not None and not isinstance(W_groups, int) and \
            W_groups.numel() < qmm_weight_bytes(N, K):
        raise ValueError("W_groups has fewer than N*K/256*144 bytes")


def qmm_run_nvfp4(h, x, W_groups, tensor_scale, y, M, N, K, stream=None):
    """Enqueue y = x . w^T for block-scaled FP4 weights (W_groups: uint8 device
    tensor from qmm_nvfp4_repack) with the given fp32 tensor scale on `stream`.
    Other arguments as for qmm_run."""
    _check_group_args(x, W_groups, y, M, N, K)
    return _check(load().qmm_run_nvfp4(h, _ptr(x), _ptr(W_groups), float(tensor_scale), _ptr(y),
                                       int(M), int(N), int(K), _stream(stream)))


def qmm_int4_repack(codes, scales, N, K):
    """Plain INT4 weights from the usual layout (numpy uint8 codes [N, K/2],
    two's complement, element 2i in the low nibble of byte i; uint16 binary16
    scales [N, K/128]) to the library's groups: a numpy uint8 array
    [N, K/256*144] (host memory; copy it to the device for qmm_run_int4)."""
    import numpy as np
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if codes.size != N * K // 2 or scales.size != N * K // 128:
        raise ValueError("codes must hold N*K/2 bytes and scales N*K/128 values")
    out = np.empty((int(N), int(K) // 256 * 144), dtype=np.uint8)
    _check(load().qmm_int4_repack(codes.ctypes.data, scales.ctypes.data, int(N), int(K),
                                  out.ctypes.data))
    return out


def qmm_run_int4(h, x, W_groups, y, M, N, K, stream=None):
    """Enqueue y = x . w^T for plain INT4 weights (W_groups: uint8 device tensor
    from qmm_int4_repack) on `stream`. Other arguments as for qmm_run."""
    _check_group_args(x, W_groups, y, M, N, K)
    return _check(load().qmm_run_int4(h, _ptr(x), _ptr(W_groups), _ptr(y), int(M), int(N),
                                      int(K), _stream(stream)))


def qmm_run_int4_raw(h, x_ptr, w_ptr, y_ptr, M, N, K, stream_ptr):
    """The C call with raw pointers; returns the status instead of raising."""
    return load().qmm_run_int4(h, x_ptr, w_ptr, y_ptr, M, N, K, stream_ptr)


def qmm_run_nvfp4_raw(h, x_ptr, w_ptr, tensor_scale, y_ptr, M, N, K, stream_ptr):
    """The C call with raw pointers; returns the status instead of raising."""
    return load().qmm_run_nvfp4(h, x_ptr, w_ptr, float(tensor_scale), y_ptr, M, N, K, stream_ptr)


def qmm_run_ids_raw(h, x_ptr, w_ptr, ids_ptr, E, y_ptr, M, N, K, stream_ptr):
    """The C call with raw pointers; returns the status instead of raising."""
    return load().qmm_run_ids(h, x_ptr, w_ptr, ids_ptr, E, y_ptr, M, N, K, stream_ptr)


def qmm_run_raw(h, x_ptr, w_ptr, y_ptr, M, N, K, stream_ptr):
    """The C call with raw pointers; returns the status instead of raising."""
    return int(load().qmm_run(h, x_ptr, w_ptr, y_ptr, int(M), int(N), int(K), stream_ptr))


def qmm_query_plan(h, M, N, K):
    p = qmm_plan()
    _check(load().qmm_query_plan(h, int(M), int(N), int(K), ctypes.byref(p)))
    return p.as_dict()


def qmm_query_plan_format(h, fmt, expert_slots, M, N, K):
    p = qmm_plan()
    _check(load().qmm_query_plan_format(h, int(fmt), int(expert_slots), int(M), int(N), int(K),
                                        ctypes.byref(p)))
    return p.as_dict()


def qmm_set_kernel(h, kernel):
    return _check(load().qmm_set_kernel(h, int(kernel)))


def qmm_set_shape(h, waves_per_wg=0, splits=0, grid_x=0):
    return _check(load().qmm_set_shape(h, int(waves_per_wg), int(splits), int(grid_x)))


def qmm_set_launch_events(h, start=None, stop=None):
    """Events (torch.cuda.Event or raw hipEvent_t) recorded around the kernel of
    the next launch on this handle: its own duration, without launch overhead."""
    def ev(e):
        if e is None:
            return None
        return e if isinstance(e, int) else e.cuda_event
    return _check(load().qmm_set_launch_events(h, ev(start), ev(stop)))


def qmm_set_wave_splits(h, wave_splits=0):
    return _check(load().qmm_set_wave_splits(h, int(wave_splits)))


def qmm_switch_point(h, N, K):
    return int(load().qmm_switch_point(h, int(N), int(K)))

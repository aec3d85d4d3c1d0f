"""Binding of the Gated DeltaNet recurrent update with log replay
(include/gdn.h) in libqmm.so: argument marshalling only. Every step of the
update runs in the library's kernel; there is no host fallback."""
import ctypes

from . import load as _load_lib, _check

EXPORTS = ["gdn_replay_update", "gdn_call_bytes"]

HEAD_DIM = 128  # dk = dv of the library's kernel

_done = False


def _lib():
    global _done
    lib = _load_lib()
    if not _done:
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.gdn_replay_update.argtypes = [vp] * 6 + [i64] + [vp] * 7 + [i64] * 5 + [vp]
        lib.gdn_replay_update.restype = ctypes.c_int
        lib.gdn_call_bytes.argtypes = [i64] * 7
        lib.gdn_call_bytes.restype = ctypes.c_uint64
        _done = True
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def gdn_replay_update_raw(state, k_log, v_log, gate_log, beta_log, n_log, L, q, k, v, gate,
                          beta, commit, o, B, M, H, dk, dv, stream=None):
    """Raw pointers (ints or None) in the header's order; returns the status."""
    return _lib().gdn_replay_update(state, k_log, v_log, gate_log, beta_log, n_log, int(L), q, k,
                                    v, gate, beta, commit, o, int(B), int(M), int(H), int(dk),
                                    int(dv), stream)


def gdn_replay_update(state, log, n_log, new, o, commit=None, stream=None):
    """Device tensors: state [B,H,dk,dv] fp32 (updated in place where commit
    > 0); log: dict of k [B,L,H,dk], v [B,L,H,dv], gate, beta [B,L,H] (or
    None); n_log: int32 [B] (or None without a log); new: dict of q, k
    [B,M,H,dk], v [B,M,H,dv], gate, beta [B,M,H]; o: [B,M,H,dv]; commit:
    int32 [B] or None. stream: a torch stream (default: the current one)."""
    import torch
    B, H, dk, dv = state.shape
    M = new["k"].shape[1] if new is not None else 0
    L = log["k"].shape[1] if log is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream()
    lg = log or {}
    nw = new or {}
    rc = gdn_replay_update_raw(
        _ptr(state), _ptr(lg.get("k")), _ptr(lg.get("v")), _ptr(lg.get("gate")),
        _ptr(lg.get("beta")), _ptr(n_log), L, _ptr(nw.get("q")), _ptr(nw.get("k")),
        _ptr(nw.get("v")), _ptr(nw.get("gate")), _ptr(nw.get("beta")), _ptr(commit), _ptr(o),
        B, M, H, dk, dv, ctypes.c_void_p(stream.cuda_stream))
    return _check(rc)


def gdn_call_bytes(B, M, H, dk, dv, log_rows, committing):
    return int(_lib().gdn_call_bytes(int(B), int(M), int(H), int(dk), int(dv), int(log_rows),
                                     int(committing)))

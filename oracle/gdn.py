"""ORACLE -- test infrastructure only (see oracle/__init__.py): the recurrent
update of a Gated DeltaNet layer with the replay of a row log, in binary64.

What the pages fix ("sixi-asi 0.11", section "A log instead of snapshots"):
the update of a layer's recurrent state is a function of the previous state
and four per-row inputs, key, value, gate and beta; a sequence keeps one base
state and the inputs of its last few rows, and a rollback replays the kept
rows on top of the base state inside the kernel that processes the new rows.
48 of the model's 64 layers are such layers, with 3.1 MB of state each, and a
snapshot after every row cost 144 MiB per row per sequence (same page,
section "What changed"): 48 x 3 MiB, so a layer's state is 3 MiB, i.e. 48
heads of 128 x 128 binary32 values (a reading; the head geometry is not on
the pages).

What the pages do not give is the update itself. It is taken from the Gated
DeltaNet paper (Yang, Kautz and Hatamizadeh, "Gated Delta Networks: Improving
Mamba2 with Delta Rule", ICLR 2025, the gated delta rule): per head, with the
state S a dv x dk matrix,

    S_t = S_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T,
    o_t = S_t q_t,

alpha_t in (0, 1] the gate (decay), beta_t in (0, 1) the write strength, k_t
of unit norm. Against the pages this oracle is therefore "parity unpinned":
its pins (tests/test_oracle_gdn.py) are the mathematics of the rule (pure
decay at beta = 0, exact overwrite of orthonormal keys at alpha = beta = 1,
the rule as a gradient step on 1/2 |S k - v|^2, the delta rule's one-step
closed form, the state layout) and the log bookkeeping (a replay split by a
commit equals the whole replay, bitwise).

The call's semantics (a reading): for sequence b the state starts from its
base state; the first n_log[b] rows of its log are applied (no outputs), then
its M new rows, each followed by its output o_t = S_t q_t; after the first
commit[b] rows of that walk (log rows first) the state at that point replaces
the base state (commit 0: the base state is unchanged).

Layout: state [B][H][dk][dv], element [b, h, e, i] = S_bh[i, e] (key index
outer, value index inner); log k [B][L][H][dk], v [B][L][H][dv], gate and
beta [B][L][H]; new rows q, k [B][M][H][dk], v [B][M][H][dv], gate, beta
[B][M][H]; outputs o [B][M][H][dv].
"""
import numpy as np

U32 = 2.0 ** -24  # unit roundoff of binary32


def step(S, k, v, alpha, beta):
    """One row of the gated delta rule on a dv x dk state (binary64)."""
    dk = S.shape[1]
    k = np.asarray(k, dtype=np.float64)
    A = float(alpha) * (np.eye(dk) - float(beta) * np.outer(k, k))
    return S @ A + float(beta) * np.outer(np.asarray(v, dtype=np.float64), k)


def replay_update(state, log, n_log, new, commit=None):
    """The whole call in binary64. state: [B,H,dk,dv]; log: dict k, v, gate,
    beta with a row axis of length L (or None); n_log: [B] ints; new: dict q,
    k, v, gate, beta with M rows; commit: [B] ints or None.

    Returns (o [B,M,H,dv], base [B,H,dk,dv] after the commit, bound_o
    [B,M,H,dv], bound_s [B,H,dk,dv], rows [B]): bound_o and bound_s are the
    magnitudes the binary32 error gate scales (see gate_o / gate_s), rows the
    rows each sequence applied."""
    state = np.asarray(state, dtype=np.float64)
    B, H, dk, dv = state.shape
    M = new["k"].shape[1]
    o = np.zeros((B, M, H, dv))
    bound_o = np.zeros((B, M, H, dv))
    base = state.copy()
    bound_s = np.zeros((B, H, dk, dv))
    rows = np.zeros(B, dtype=np.int64)
    for b in range(B):
        nl = int(n_log[b]) if log is not None else 0
        c = 0 if commit is None else int(commit[b])
        T = nl + M
        for h in range(H):
            S = state[b, h].T.copy()  # dv x dk
            R = np.sqrt((S * S).sum(axis=1))  # running magnitude per value row
            walk = [(log, r) for r in range(nl)] + [(new, t) for t in range(M)]
            for idx, (src, r) in enumerate(walk):
                k = src["k"][b, r, h].astype(np.float64)
                v = src["v"][b, r, h].astype(np.float64)
                a, bt = float(src["gate"][b, r, h]), float(src["beta"][b, r, h])
                S = step(S, k, v, a, bt)
                R = np.maximum(R, np.sqrt((S * S).sum(axis=1)) + abs(bt) * np.abs(v))
                if src is new:
                    q = new["q"][b, r, h].astype(np.float64)
                    o[b, r, h] = S @ q
                    bound_o[b, r, h] = R * np.sqrt(q @ q) + np.abs(S) @ np.abs(q)
                if idx + 1 == c:
                    base[b, h] = S.T
                    bound_s[b, h] = np.broadcast_to(R, (dk, dv))
        rows[b] = T
    return o, base, bound_o, bound_s, rows


def eps(rows, dk):
    """Relative error allowance of a binary32 evaluation after `rows` rows:
    (rows + 1) (dk + 8) u. Each row's dot product of length dk errs by at most
    gamma_dk = dk u / (1 - dk u) of the sum of its terms' magnitudes, the decay
    and the write add a few roundings per element, and the rule is a
    contraction for unit keys (alpha <= 1, the eigenvalues of I - beta k k^T
    lie in [1 - beta, 1]), so earlier errors do not grow; the allowance adds
    one such error per row applied."""
    return (np.asarray(rows, dtype=np.float64) + 1.0) * (dk + 8) * U32

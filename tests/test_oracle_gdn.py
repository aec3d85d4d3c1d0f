"""Pins of the recurrent-update oracle (oracle/gdn.py) by the mathematics of
the gated delta rule and by the log bookkeeping. Against the pages the rule is
parity unpinned (the pages give its inputs, not its equation)."""
import numpy as np
import pytest

import synth
from oracle import gdn


def rows(B, R, H, dk, dv, tensor, queries=True):
    return {k: v.astype(np.float64) for k, v in synth.gdn_rows(B, R, H, dk, dv, tensor, queries=queries).items()}


def test_beta_zero_is_pure_decay():
    # beta = 0: S_t = (alpha_1 ... alpha_t) S_0 whatever the keys and values
    B, H, dk, dv, L, M = 2, 3, 16, 12, 4, 3
    state = synth.gdn_state(B, H, dk, dv, tensor=1).astype(np.float64)
    log, new = rows(B, L, H, dk, dv, 2, queries=False), rows(B, M, H, dk, dv, 3)
    log["beta"][:] = 0.0
    new["beta"][:] = 0.0
    n_log = np.array([4, 2])
    commit = n_log + M
    o, base, _, _, _ = gdn.replay_update(state, log, n_log, new, commit)
    for b in range(B):
        for h in range(H):
            P = np.prod(log["gate"][b, :n_log[b], h])
            for t in range(M):
                P *= new["gate"][b, t, h]
                # o_t[i] = sum_e S[i, e] q[e], with S[i, e] stored at state[b, h, e, i]
                want = P * np.einsum("ei,e->i", state[b, h], new["q"][b, t, h])
                assert np.allclose(o[b, t, h], want, rtol=1e-13, atol=1e-15)
            assert np.allclose(base[b, h], P * state[b, h], rtol=1e-13, atol=1e-15)


def test_orthonormal_keys_are_overwritten_exactly():
    # alpha = beta = 1 with orthonormal keys: each write makes S k_j = v_j and
    # leaves the earlier keys' values in place (k_i orthogonal to k_j)
    B, H, dk, dv, M = 1, 2, 16, 10, 6
    rng = np.random.default_rng(3)
    state = synth.gdn_state(B, H, dk, dv, tensor=4).astype(np.float64)
    new = rows(B, M, H, dk, dv, 5)
    for h in range(H):
        Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        new["k"][0, :, h] = Q[:M]
    new["gate"][:] = 1.0
    new["beta"][:] = 1.0
    _, base, _, _, _ = gdn.replay_update(state, None, [0], new, [M])
    for h in range(H):
        S = base[0, h].T
        for j in range(M):
            assert np.allclose(S @ new["k"][0, j, h], new["v"][0, j, h], atol=1e-12)


def test_rule_is_a_gradient_step_on_the_regression_loss():
    # alpha = 1: S' = S - beta * dL/dS with L(S) = 1/2 |S k - v|^2; the gradient
    # by central differences (exact for a quadratic up to rounding)
    rng = np.random.default_rng(7)
    dv, dk = 5, 7
    S = rng.standard_normal((dv, dk))
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(dv)
    beta = 0.37

    def loss(X):
        r = X @ k - v
        return 0.5 * r @ r

    grad = np.zeros_like(S)
    h = 1e-3
    for i in range(dv):
        for e in range(dk):
            d = np.zeros_like(S)
            d[i, e] = h
            grad[i, e] = (loss(S + d) - loss(S - d)) / (2 * h)
    assert np.allclose(gdn.step(S, k, v, 1.0, beta), S - beta * grad, atol=1e-9)
    # the gate scales the old state but not the new write
    alpha = 0.6
    assert np.allclose(gdn.step(S, k, v, alpha, beta),
                       alpha * (S - beta * np.outer(S @ k, k)) + beta * np.outer(v, k), atol=1e-12)


def test_one_step_closed_forms_and_layout():
    B, H, dk, dv = 1, 1, 8, 6
    new = rows(B, 1, H, dk, dv, 9)
    # from a zero state one row writes beta v k^T: o = beta v (k . q)
    o, _, _, _, _ = gdn.replay_update(np.zeros((B, H, dk, dv)), None, [0], new)
    k, q, v = new["k"][0, 0, 0], new["q"][0, 0, 0], new["v"][0, 0, 0]
    assert np.allclose(o[0, 0, 0], new["beta"][0, 0, 0] * v * (k @ q), atol=1e-15)
    # a state with the single entry S[i=4, e=2] = 1 (stored at [.., 2, 4]) under
    # beta = 0, alpha = 1 reads out q[2] into output 4 only
    state = np.zeros((B, H, dk, dv))
    state[0, 0, 2, 4] = 1.0
    new["beta"][:] = 0.0
    new["gate"][:] = 1.0
    o, _, _, _, _ = gdn.replay_update(state, None, [0], new)
    want = np.zeros(dv)
    want[4] = q[2]
    assert np.array_equal(o[0, 0, 0], want)


def test_replay_split_by_a_commit_equals_the_whole_replay():
    # one call over 5 log rows and 3 new rows, against a call that commits
    # after 6 rows followed by one that replays the 7th row from the log and
    # takes the 8th as its new row: same outputs and base state, bitwise
    B, H, dk, dv = 2, 2, 16, 12
    state = synth.gdn_state(B, H, dk, dv, tensor=11).astype(np.float64)
    log, new = rows(B, 5, H, dk, dv, 12, queries=False), rows(B, 3, H, dk, dv, 13)
    n_log = np.array([5, 5])
    o_all, base_all, _, _, _ = gdn.replay_update(state, log, n_log, new, [8, 8])
    o1, base6, _, _, _ = gdn.replay_update(state, log, n_log, new, [6, 6])
    log2 = {k: new[k][:, 1:2] for k in ("k", "v", "gate", "beta")}
    new2 = {k: new[k][:, 2:3] for k in ("q", "k", "v", "gate", "beta")}
    o2, base8, _, _, _ = gdn.replay_update(base6, log2, [1, 1], new2, [2, 2])
    assert np.array_equal(base8, base_all)
    assert np.array_equal(o2[:, 0], o_all[:, 2])
    assert np.array_equal(o1, o_all)
    # commit 0 leaves the base state as it was; a ragged log applies its own count
    _, base0, _, _, nrows = gdn.replay_update(state, log, [5, 2], new, [0, 0])
    assert np.array_equal(base0, state) and list(nrows) == [8, 5]


def test_replay_equals_sequential_steps():
    # the call's walk is the rows in order: log rows, then the new rows
    B, H, dk, dv = 1, 1, 16, 12
    state = synth.gdn_state(B, H, dk, dv, tensor=21).astype(np.float64)
    log, new = rows(B, 4, H, dk, dv, 22, queries=False), rows(B, 2, H, dk, dv, 23)
    o, base, _, _, _ = gdn.replay_update(state, log, [3], new, [5])
    S = state[0, 0].T
    for r in range(3):
        S = gdn.step(S, log["k"][0, r, 0], log["v"][0, r, 0], log["gate"][0, r, 0], log["beta"][0, r, 0])
    S = gdn.step(S, new["k"][0, 0, 0], new["v"][0, 0, 0], new["gate"][0, 0, 0], new["beta"][0, 0, 0])
    assert np.array_equal(o[0, 0, 0], S @ new["q"][0, 0, 0])
    S = gdn.step(S, new["k"][0, 1, 0], new["v"][0, 1, 0], new["gate"][0, 1, 0], new["beta"][0, 1, 0])
    assert np.array_equal(o[0, 1, 0], S @ new["q"][0, 1, 0])
    assert np.array_equal(base[0, 0], S.T)


def test_error_allowance():
    assert gdn.eps(0, 128) == pytest.approx(136 * 2.0 ** -24)
    assert gdn.eps(15, 128) == pytest.approx(16 * 136 * 2.0 ** -24)


def test_input_recipe():
    r = synth.gdn_rows(2, 3, 4, 128, 128, tensor=5)
    assert np.allclose(np.linalg.norm(r["k"].astype(np.float64), axis=-1), 1.0, atol=1e-6)
    assert np.allclose(np.linalg.norm(r["q"].astype(np.float64), axis=-1), 128 ** -0.5, atol=1e-7)
    assert r["gate"].min() >= 0.85 and r["gate"].max() < 1.0
    assert r["beta"].min() >= 0.05 and r["beta"].max() < 0.95
    s = synth.gdn_state(1, 48, 128, 128, tensor=1)
    assert s.nbytes == 3 * 2 ** 20  # 3 MiB per sequence and layer

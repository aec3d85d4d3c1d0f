"""GPU parity of the recurrent update with log replay (include/gdn.h) against
the binary64 oracle (oracle/gdn.py), through the C ABI.

Gate per output element after T rows: |o - o_ref| <= (T + 1)(dk + 8) 2^-24 *
(R |q| + sum_e |S_ie q_e|) with R the row's largest |S_i.| + beta |v_i| along
the walk (oracle.gdn.eps and the bounds replay_update returns); the committed
state likewise. States of sequences that do not commit must come back
bit-identical, and repeated calls must agree bitwise. Inputs: the seeded
recipe of synth.gdn_rows / synth.gdn_state.
"""
import numpy as np
import pytest

import synth
from oracle import gdn as ogdn

torch = pytest.importorskip("torch")
import skinny_bit_block_amd as sbb  # noqa: E402
from skinny_bit_block_amd import gdn  # noqa: E402

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def make(B, H, L, M, tensor):
    state = synth.gdn_state(B, H, D, D, tensor=tensor)
    log = synth.gdn_rows(B, L, H, D, D, tensor=tensor + 1, queries=False) if L > 0 else None
    new = synth.gdn_rows(B, M, H, D, D, tensor=tensor + 2) if M > 0 else None
    return state, log, new


def dev(d):
    return None if d is None else {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in d.items()}


def run(state, log, n_log, new, commit, B, H, M):
    st = torch.from_numpy(state.copy()).cuda()
    o = torch.full((B, M, H, D), float("nan"), device="cuda") if M > 0 else None
    nl = torch.tensor(np.asarray(n_log, dtype=np.int32)).cuda() if log is not None else None
    cm = torch.tensor(np.asarray(commit, dtype=np.int32)).cuda() if commit is not None else None
    gdn.gdn_replay_update(st, dev(log), nl, dev(new), o, commit=cm)
    torch.cuda.synchronize()
    return st.cpu().numpy(), (o.cpu().numpy() if o is not None else None)


def check(state, log, n_log, new, commit, st_gpu, o_gpu, what):
    """Compare with the oracle at the clamped n_log / commit the kernel uses."""
    B, H = state.shape[:2]
    M = new["k"].shape[1] if new is not None else 0
    L = log["k"].shape[1] if log is not None else 0
    nl = np.clip(np.asarray(n_log if log is not None else [0] * B), 0, L)
    cm = np.clip(np.asarray(commit if commit is not None else [0] * B), 0, nl + M)
    empty = {"q": np.zeros((B, 0, H, D)), "k": np.zeros((B, 0, H, D)), "v": np.zeros((B, 0, H, D)),
             "gate": np.zeros((B, 0, H)), "beta": np.zeros((B, 0, H))}
    o_ref, base_ref, bo, bs, _ = ogdn.replay_update(state, log, nl, new if new is not None else empty, cm)
    if M > 0:
        assert np.isfinite(o_gpu).all(), what
        rows = nl[:, None, None, None] + np.arange(1, M + 1)[None, :, None, None]
        tol = ogdn.eps(rows, D) * bo
        err = np.abs(o_gpu.astype(np.float64) - o_ref)
        bad = err > tol
        assert not bad.any(), "%s: %d outputs outside the gate, worst err/tol %.3g" % (
            what, bad.sum(), (err / np.maximum(tol, 1e-300)).max())
    for b in range(B):
        if cm[b] == 0:
            assert np.array_equal(st_gpu[b], state[b]), "%s: sequence %d without commit changed" % (what, b)
        else:
            tol = ogdn.eps(cm[b], D) * bs[b]
            err = np.abs(st_gpu[b].astype(np.float64) - base_ref[b])
            assert (err <= tol).all(), "%s: state of sequence %d, worst err/tol %.3g" % (
                what, b, (err / np.maximum(tol, 1e-300)).max())


@pytest.mark.parametrize("B,H,L,M,n_log,commit", [
    (3, 2, 6, 4, [6, 0, 3], [0, 2, 7]),       # ragged logs; commits inside the new rows and at the end
    (2, 3, 5, 3, [5, 5], [3, 8]),             # commit inside the log
    (1, 1, 0, 5, None, [5]),                  # no log
    (2, 2, 4, 0, [4, 2], [4, 1]),             # replay and commit only, no outputs
    (2, 2, 3, 2, [3, 1], None),               # no commit: states unchanged
    (4, 48, 8, 4, [0, 3, 8, 5], [0, 7, 12, 5]),  # a layer's 48 heads
    (2, 2, 64, 8, [64, 33], [50, 72]),        # long logs (72-row walks)
    (1, 1, 1, 1, [1], [2]),                   # one head, one kept row, one new row
    (5, 1, 2, 1, [0, 1, 2, 0, 2], [1, 0, 3, 0, 1]),  # single-row walks, ragged
])
def test_parity(B, H, L, M, n_log, commit):
    state, log, new = make(B, H, L, M, tensor=100 + B * 7 + H + L + M)
    st, o = run(state, log, n_log, new, commit, B, H, M)
    check(state, log, n_log, new, commit, st, o, "B=%d H=%d L=%d M=%d" % (B, H, L, M))


def test_out_of_range_counts_are_clamped():
    B, H, L, M = 4, 2, 3, 2
    state, log, new = make(B, H, L, M, tensor=300)
    n_log, commit = [7, -2, 3, 1], [-5, 99, 4, 2]
    st, o = run(state, log, n_log, new, commit, B, H, M)
    check(state, log, n_log, new, commit, st, o, "clamped")


@pytest.mark.parametrize("kind", ["small", "zero", "mixed"])
def test_small_gates_fold_the_scaled_state(kind):
    # gate products far below 2^-64 within one walk (folds), gates of exactly
    # zero (the floor), and a mix with ordinary gates
    B, H, L, M = 2, 2, 12, 6
    state, log, new = make(B, H, L, M, tensor=400)
    rng = np.random.default_rng(5)
    for d in (log, new):
        if kind == "small":
            d["gate"][:] = 1e-3
        elif kind == "zero":
            d["gate"][:, ::3] = 0.0
        else:
            d["gate"][:] = np.where(rng.random(d["gate"].shape) < 0.3, 1e-6, d["gate"]).astype(np.float32)
    n_log, commit = [12, 7], [15, 4]
    st, o = run(state, log, n_log, new, commit, B, H, M)
    check(state, log, n_log, new, commit, st, o, "gates " + kind)


def test_bitwise_repeatable():
    B, H, L, M = 2, 4, 5, 3
    state, log, new = make(B, H, L, M, tensor=500)
    a = run(state, log, [5, 2], new, [6, 3], B, H, M)
    b = run(state, log, [5, 2], new, [6, 3], B, H, M)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_layer_of_32_sequences():
    # the benchmarked shape: 32 sequences x 48 heads (3 MiB of state each),
    # 4 new rows, logs of 0..8 kept rows folded into the base state; the
    # oracle checks a sample of (sequence, head) pairs, every output is finite
    # and the states of the sequences without a log come back unchanged
    B, H, L, M = 32, 48, 8, 4
    state, log, new = make(B, H, L, M, tensor=600)
    n_log = [b % 9 for b in range(B)]
    commit = list(n_log)
    st, o = run(state, log, n_log, new, commit, B, H, M)
    assert np.isfinite(o).all() and np.isfinite(st).all()
    for b in range(B):
        if commit[b] == 0:
            assert np.array_equal(st[b], state[b])
    pick_b = [0, 5, 8, 17, 31]
    pick_h = [0, 13, 47]
    sub = lambda d: None if d is None else {k: v[pick_b][:, :, pick_h] for k, v in d.items()}
    check(state[pick_b][:, pick_h], sub(log), [n_log[b] for b in pick_b], sub(new),
          [commit[b] for b in pick_b], st[pick_b][:, pick_h], o[pick_b][:, :, pick_h], "32 x 48")


def test_graph_replays_match_eager_calls():
    # a captured call replayed several times (with eager work and syncs in
    # between) against the same calls made eagerly on a second copy of the
    # state: committing calls change the state each time, so every replay's
    # outputs and state must equal the matching eager call's, bitwise
    B, H, L, M = 3, 4, 4, 3
    state, log, new = make(B, H, L, M, tensor=700)
    n_log = torch.tensor([4, 1, 3], dtype=torch.int32, device="cuda")
    commit = torch.tensor([5, 0, 6], dtype=torch.int32, device="cuda")
    lg, nw = dev(log), dev(new)
    st_g = torch.from_numpy(state.copy()).cuda()
    st_e = torch.from_numpy(state.copy()).cuda()
    o_g = torch.zeros((B, M, H, D), device="cuda")
    o_e = torch.zeros((B, M, H, D), device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        gdn.gdn_replay_update(st_g, lg, n_log, nw, o_g, commit=commit, stream=side)
    torch.cuda.synchronize()
    # capture does not run the call: both copies are still the base state
    assert torch.equal(st_g, st_e)
    for step in range(4):
        g.replay()
        torch.cuda.synchronize()
        gdn.gdn_replay_update(st_e, lg, n_log, nw, o_e, commit=commit)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), step
        assert torch.equal(st_g, st_e), step
        st_e.add_(0.0)  # eager work between replays
    assert not torch.equal(st_g.cpu(), torch.from_numpy(state))  # the commits moved it


def draw_gdn_cases(n=80, seed=20261205):
    """Seeded (B, H, L, M, n_log, commit, gate regime) cases: ragged and
    out-of-range log counts and commits, empty logs and calls without new
    rows, and ordinary, tiny and zero gates."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, H = int(rng.integers(1, 6)), int(rng.integers(1, 4))
        L, M = int(rng.choice([0, 1, 3, 8, 20])), int(rng.choice([0, 1, 2, 4, 7]))
        n_log = [int(v) for v in rng.integers(-2, L + 3, B)] if L > 0 else None
        commit = [int(v) for v in rng.integers(-2, L + M + 3, B)] if rng.random() < 0.8 else None
        out.append((B, H, L, M, n_log, commit, str(rng.choice(["plain", "plain", "small", "zero"]))))
    return out


GDN_CASES = draw_gdn_cases()


@pytest.mark.parametrize("i", range(len(GDN_CASES)))
def test_seeded_sweep(i):
    B, H, L, M, n_log, commit, gates = GDN_CASES[i]
    state, log, new = make(B, H, L, M, tensor=1000 + 10 * i)
    for d in (log, new):
        if d is None:
            continue
        if gates == "small":
            d["gate"][:] = 1e-3
        elif gates == "zero":
            d["gate"][:, ::2] = 0.0
    st, o = run(state, log, n_log, new, commit, B, H, M)
    check(state, log, n_log, new, commit, st, o,
          "sweep %d: B=%d H=%d L=%d M=%d n_log=%s commit=%s gates=%s" % (i, B, H, L, M, n_log, commit, gates))

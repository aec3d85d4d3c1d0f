"""GPU parity of the expert-indexed product (qmm_run_ids) against oracle.qmm_ids."""
import numpy as np
import pytest

import oracle
import skinny_bit_block_amd as sbb
import synth

torch = pytest.importorskip("torch")
TOL = 2e-3

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    handle = sbb.qmm_create(0)
    yield handle
    sbb.qmm_destroy(handle)


def experts(E, N, K, base):
    return np.concatenate([synth.weights(N, K, tensor=base + e).reshape(-1) for e in range(E)])


def run_ids(h, x, W, ids, E, N, K, shape=(0, 0, 0), wave_splits=0, fill=7.0):
    M = x.shape[0]
    sbb.qmm_set_shape(h, *shape)
    sbb.qmm_set_wave_splits(h, wave_splits)
    try:
        xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        Wd = torch.from_numpy(np.ascontiguousarray(W)).cuda()
        idd = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
        y = torch.full((M, N), fill, dtype=torch.float32, device="cuda")
        sbb.qmm_run_ids(h, xd, Wd, idd, E, y, M, N, K)
        torch.cuda.synchronize()
        return y.cpu().numpy()
    finally:
        sbb.qmm_set_shape(h, 0, 0, 0)
        sbb.qmm_set_wave_splits(h, 0)


def check_ids(y, x, W, ids, E, N, K, what):
    yref, aref, written = oracle.qmm_ids(x, W, ids, E, N, K)
    assert np.all(y[~written] == 7.0), what + ": a row with an invalid id was written"
    yw, rw, aw = y[written].astype(np.float64), yref[written], aref[written]
    assert np.all(np.isfinite(yw)), what
    bad = np.abs(yw - rw) > TOL * aw
    assert not bad.any(), "%s: %d elements outside the gate" % (what, bad.sum())


def id_pattern(kind, M, E, rng):
    if kind == "random":
        return rng.integers(0, E, M)
    if kind == "same":
        return np.full(M, E - 1)
    if kind == "distinct":
        return rng.permutation(E)[:M] if M <= E else np.arange(M) % E
    if kind == "invalid":
        v = rng.integers(0, E, M)
        v[::3] = -1
        if M > 1:
            v[1] = E + 5
        return v
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["random", "same", "distinct", "invalid"])
@pytest.mark.parametrize("M,E", [(1, 4), (3, 4), (8, 8), (8, 64), (17, 6), (32, 5)])
def test_ids_parity(h, M, E, kind):
    N, K = 300, 1280
    rng = np.random.default_rng(1000 * M + E)
    ids = id_pattern(kind, M, E, rng)
    W = experts(E, N, K, 800 + E)
    x = synth.acts(M, K, tensor=810 + M)
    y = run_ids(h, x, W, ids, E, N, K)
    check_ids(y, x, W, ids, E, N, K, "M=%d E=%d %s" % (M, E, kind))


@pytest.mark.parametrize("M,E,N,K", [(7, 4, 5, 1 << 20), (32, 3, 3, 1 << 18), (2, 2, 17, 1 << 19)])
def test_ids_long_k(h, M, E, N, K):
    # K far beyond the workloads' (thousands of K slices per expert slot); the
    # host address replay walks the same plans
    rng = np.random.default_rng(M + E)
    ids = rng.integers(0, E, M)
    W = experts(E, N, K, 870 + E)
    x = synth.acts(M, K, tensor=880 + M)
    y = run_ids(h, x, W, ids, E, N, K)
    check_ids(y, x, W, ids, E, N, K, "long K: M=%d E=%d N=%d K=%d" % (M, E, N, K))


@pytest.mark.parametrize("shape,wsplit", [((4, 3, 0), 0), ((4, 2, 2), 2), ((2, 1, 1), 0),
                                          ((8, 5, 0), 0), ((4, 4, 0), 4)])
def test_ids_launch_shapes(h, shape, wsplit):
    M, E, N, K = 12, 7, 1000, 2560
    rng = np.random.default_rng(7)
    ids = rng.integers(0, E, M)
    W = experts(E, N, K, 830)
    x = synth.acts(M, K, tensor=840)
    y = run_ids(h, x, W, ids, E, N, K, shape=shape, wave_splits=wsplit)
    check_ids(y, x, W, ids, E, N, K, "shape=%s wave_splits=%d" % (shape, wsplit))


def test_ids_repeat_is_bitwise_identical(h):
    M, E, N, K = 9, 5, 700, 1536
    ids = np.array([3, 1, 3, 0, 4, 4, 1, 2, 3])
    W = experts(E, N, K, 850)
    x = synth.acts(M, K, tensor=860)
    y1 = run_ids(h, x, W, ids, E, N, K, shape=(4, 3, 0))
    y2 = run_ids(h, x, W, ids, E, N, K, shape=(4, 3, 0))
    assert np.array_equal(y1, y2)
    check_ids(y1, x, W, ids, E, N, K, "repeat")

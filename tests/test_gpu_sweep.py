"""Seeded sweeps of forced launch shapes over ragged small matrices on the GPU,
in the three weight formats and for expert-indexed calls, against the
binary64 oracles.

The cases are drawn the way the host address replay draws its own seeded
sweep (tests/test_address_sim.py): N with ragged last row tiles, K of 1..17
super-blocks (partial last stages of every length), 1..32 rows, either
kernel, and forced waves, K slices, grids and in-workgroup slices. Each case
takes the plan the device handle makes (its grid capped at the device's
residency), replays that plan's load addresses on the host, and only then
launches; the output is checked against the oracle at the product's gate,
|y - y_ref| <= 2e-3 * sum_k |w x|, and must be finite everywhere (y starts as
NaN, so a tile left unwritten fails).
"""
import numpy as np
import pytest

import oracle
import synth
import test_address_sim as addr
from oracle import int4 as oint4
from oracle import nvfp4 as ofp4

torch = pytest.importorskip("torch")
import skinny_bit_block_amd as sbb  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 2e-3
SEED = 20261202
NS = [1, 3, 15, 16, 17, 33, 129, 300, 333, 1000, 2047]
KS = [256 * b for b in (1, 2, 3, 4, 5, 6, 7, 9, 10, 13, 17)]


def draw_cases(n=400, seed=20261203):
    """(fmt, M, N, K, kernel, (waves, splits, grid), wsplit) tuples that the
    planner accepts (a planning-only handle: the same checks as a device's)."""
    rng = np.random.default_rng(seed)
    h = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    out = []
    try:
        while len(out) < n:
            N, K = int(rng.choice(NS)), int(rng.choice(KS))
            M = int(rng.integers(1, 33))
            kernel = int(rng.choice([sbb.KERNEL_VECTOR, sbb.KERNEL_TILED]))
            fmt = int(rng.choice([0, 1, 2])) if kernel == sbb.KERNEL_TILED else 0
            shape = (int(rng.integers(1, 9)), int(rng.integers(0, K // 256 + 1)),
                     int(rng.choice([0, 0, 1, 2, 3, 7])))
            wsplit = int(rng.choice([0, 1, 1, 2, 3, 4, 8]))
            if addr.plan(h, fmt, 0, M, N, K, kernel, shape, wsplit) is not None:
                out.append((fmt, M, N, K, kernel, shape, wsplit))
    finally:
        sbb.qmm_destroy(h)
    return out


NCASES = 400
_cases = []


def cases():
    if not _cases:
        _cases.extend(draw_cases(NCASES))
    return _cases


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    handle = sbb.qmm_create(0)
    yield handle
    sbb.qmm_destroy(handle)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1) if a.dtype == np.uint8
                            else np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("i", range(NCASES))
def test_forced_shape_sweep(h, i):
    fmt, M, N, K, kernel, shape, wsplit = cases()[i]
    what = "fmt=%d M=%d N=%d K=%d kernel=%d shape=%s wsplit=%d" % (fmt, M, N, K, kernel, shape, wsplit)
    tensor = 5000 + 10 * i
    x = synth.acts(M, K, tensor=tensor, seed=SEED)
    if fmt == 0:
        W = synth.weights(N, K, tensor=tensor + 1, seed=SEED)
        yref, aref = oracle.qmm(x, W, N, K)
    elif fmt == 1:
        elems, scales = synth.nvfp4(N, K, tensor=tensor + 1, seed=SEED)
        W = sbb.qmm_nvfp4_repack(elems, scales, N, K)
        yref, aref = ofp4.qmm_nvfp4(x, elems, scales, 0.37, N, K)
    else:
        codes, scales = synth.int4(N, K, tensor=tensor + 1, seed=SEED)
        W = sbb.qmm_int4_repack(codes, scales, N, K)
        yref, aref = oint4.qmm_int4(x, codes, scales, N, K)
    sbb.qmm_set_kernel(h, kernel)
    sbb.qmm_set_shape(h, *shape)
    sbb.qmm_set_wave_splits(h, wsplit)
    try:
        p = sbb.qmm_query_plan_format(h, fmt, 0, M, N, K)
        addr.replay(p, M, N, K)  # every load of the launch stays inside W and x
        xd, Wd = dev(x), dev(W)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        if fmt == 0:
            sbb.qmm_run(h, xd, Wd, y, M, N, K)
        elif fmt == 1:
            sbb.qmm_run_nvfp4(h, xd, Wd, 0.37, y, M, N, K)
        else:
            sbb.qmm_run_int4(h, xd, Wd, y, M, N, K)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
    finally:
        sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)
        sbb.qmm_set_shape(h, 0, 0, 0)
        sbb.qmm_set_wave_splits(h, 0)
    assert np.isfinite(y).all(), what
    err = np.abs(y.astype(np.float64) - yref)
    bad = err > TOL * aref
    assert not bad.any(), "%s: %d of %d outside the gate, worst err/A %.3g" % (
        what, int(bad.sum()), bad.size, float((err / np.maximum(aref, 1e-300)).max()))


# ------------------------------------------------------------- expert-indexed

ID_KINDS = ["random", "same", "distinct", "invalid"]
NIDS = 150
_id_cases = []


def id_pattern(kind, M, E, rng):
    if kind == "random":
        return rng.integers(0, E, M)
    if kind == "same":
        return np.full(M, int(rng.integers(0, E)))
    if kind == "distinct":
        return rng.permutation(E)[:M] if M <= E else np.arange(M) % E
    v = rng.integers(0, E, M)  # invalid ids (negative, past E) write nothing
    v[::3] = -1
    if M > 1:
        v[1] = E + 5
    return v


def draw_id_cases(n=NIDS, seed=20261204):
    """(M, N, K, E, ids, (waves, splits, grid), wsplit) that the planner accepts
    for an expert-indexed call (slots = min(M, E))."""
    rng = np.random.default_rng(seed)
    h = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    out = []
    try:
        while len(out) < n:
            N, K = int(rng.choice(NS)), int(rng.choice(KS[:9]))
            M = int(rng.integers(1, 33))
            E = int(rng.choice([1, 2, 3, 5, 8, 17]))
            ids = id_pattern(str(rng.choice(ID_KINDS)), M, E, rng).astype(np.int32)
            shape = (int(rng.integers(1, 9)), int(rng.integers(0, K // 256 + 1)),
                     int(rng.choice([0, 0, 1, 2, 3, 7])))
            wsplit = int(rng.choice([0, 1, 1, 2, 3, 4, 8]))
            if addr.plan(h, sbb.FORMAT_KQUANT, min(M, E), M, N, K, sbb.KERNEL_AUTO, shape,
                         wsplit) is not None:
                out.append((M, N, K, E, ids, shape, wsplit))
    finally:
        sbb.qmm_destroy(h)
    return out


def id_cases():
    if not _id_cases:
        _id_cases.extend(draw_id_cases())
    return _id_cases


@pytest.mark.parametrize("i", range(NIDS))
def test_expert_indexed_sweep(h, i):
    M, N, K, E, ids, shape, wsplit = id_cases()[i]
    what = "M=%d N=%d K=%d E=%d ids=%s shape=%s wsplit=%d" % (M, N, K, E, ids.tolist(), shape, wsplit)
    tensor = 9000 + 40 * i
    x = synth.acts(M, K, tensor=tensor, seed=SEED)
    W = np.concatenate([synth.weights(N, K, tensor=tensor + 1 + e, seed=SEED).reshape(-1)
                        for e in range(E)])
    yref, aref, written = oracle.qmm_ids(x, W, ids, E, N, K)
    sbb.qmm_set_shape(h, *shape)
    sbb.qmm_set_wave_splits(h, wsplit)
    try:
        p = sbb.qmm_query_plan_format(h, sbb.FORMAT_KQUANT, min(M, E), M, N, K)
        # each slot stages the rows of one expert: every row count up to M
        for m in sorted({1, M} | {int((ids == e).sum()) for e in range(E) if (ids == e).any()}):
            addr.replay(p, m, N, K)
        xd, Wd = dev(x), dev(W)
        idd = torch.from_numpy(ids).cuda()
        y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
        sbb.qmm_run_ids(h, xd, Wd, idd, E, y, M, N, K)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
    finally:
        sbb.qmm_set_shape(h, 0, 0, 0)
        sbb.qmm_set_wave_splits(h, 0)
    assert np.all(y[~written] == 7.0), what + ": a row with an invalid id was written"
    yw = y[written].astype(np.float64)
    assert np.isfinite(yw).all(), what
    bad = np.abs(yw - yref[written]) > TOL * aref[written]
    assert not bad.any(), "%s: %d elements outside the gate" % (what, int(bad.sum()))

"""HIP graph capture and replay of the library's calls (the way bench.py times
the model pass): a captured sequence of products replayed several times, with
the program's own eager work and synchronizations between the replays, must
give bit-identical outputs to the same calls run eagerly every time. The
sequence covers split-K across workgroups (the per-tile arrival counters the
last wave resets in-kernel), in-workgroup K splits, both kernels, and the
expert-indexed, FP4 and INT4 instantiations; the eager results themselves are
checked against the oracles on sampled rows."""
import numpy as np
import pytest

import oracle
import synth
from oracle import int4 as i4
from oracle import nvfp4 as fp4

torch = pytest.importorskip("torch")
import skinny_bit_block_amd as sbb  # noqa: E402

pytestmark = pytest.mark.gpu

SEED = 20261202
TOL = 2e-3


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    handle = sbb.qmm_create(0)
    yield handle
    sbb.qmm_destroy(handle)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _calls(h):
    """(label, launch(stream), y, reference check) for each product."""
    out = []
    # 4.5-bit super-blocks: row-vector kernel with split-K at 1 row (5120x5120
    # takes 5 slices over 3 workgroup ranges), tiled at 8 and 16 rows
    for M, N, K, tag in ((1, 5120, 5120, 1), (8, 5120, 17408, 2), (16, 34816, 5120, 3)):
        W = synth.weights(N, K, tensor=3000 + tag, seed=SEED)
        x = synth.acts(M, K, tensor=3100 + tag, seed=SEED)
        Wd, xd = _dev(W.reshape(-1)), _dev(x)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        rows = np.r_[0:3, N // 2:N // 2 + 3, N - 3:N]

        def ref(yh, x=x, W=W, N=N, K=K, rows=rows):
            yr, ar = oracle.qmm_rows(x, W, N, K, rows)
            return yh[:, rows], yr, ar
        out.append(("q4 M=%d N=%d K=%d" % (M, N, K),
                    lambda s, Wd=Wd, xd=xd, y=y, M=M, N=N, K=K:
                    sbb.qmm_run(h, xd, Wd, y, M, N, K, stream=s), y, ref))
    # expert-indexed: 6 rows over 3 of 4 experts
    M, N, K, E = 6, 1000, 2560, 4
    Ws = [synth.weights(N, K, tensor=3200 + e, seed=SEED) for e in range(E)]
    x = synth.acts(M, K, tensor=3300, seed=SEED)
    ids = np.array([2, 0, 2, 3, 0, 2], dtype=np.int32)
    Wd = _dev(np.concatenate([w.reshape(-1) for w in Ws]))
    xd, idd = _dev(x), _dev(ids)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def ref_ids(yh, x=x, Ws=Ws, ids=ids, N=N, K=K):
        rows = np.arange(0, N, 37)
        yr = np.empty((len(ids), len(rows)))
        ar = np.empty_like(yr)
        for m, e in enumerate(ids):
            yy, aa = oracle.qmm_rows(x[m:m + 1], Ws[e], N, K, rows)
            yr[m], ar[m] = yy[0], aa[0]
        return yh[:, rows], yr, ar
    out.append(("ids", lambda s, xd=xd, Wd=Wd, idd=idd, y=y, M=M, N=N, K=K, E=E:
                sbb.qmm_run_ids(h, xd, Wd, idd, E, y, M, N, K, stream=s), y, ref_ids))
    # block-scaled FP4 and plain INT4, 7 rows
    M, N, K = 7, 3000, 5120
    elems, scales = synth.nvfp4(N, K, tensor=3400, seed=SEED)
    x = synth.acts(M, K, tensor=3401, seed=SEED)
    g4 = _dev(sbb.qmm_nvfp4_repack(elems, scales, N, K).reshape(-1))
    xd = _dev(x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def ref_fp4(yh, x=x, elems=elems, scales=scales, N=N, K=K):
        rows = np.arange(0, N, 41)
        yr, ar = fp4.qmm_nvfp4(x, elems, scales, 0.75, N, K, rows=rows)
        return yh[:, rows], yr, ar
    out.append(("fp4", lambda s, xd=xd, g4=g4, y=y, M=M, N=N, K=K:
                sbb.qmm_run_nvfp4(h, xd, g4, 0.75, y, M, N, K, stream=s), y, ref_fp4))
    codes, iscales = synth.int4(N, K, tensor=3500, seed=SEED)
    gi = _dev(sbb.qmm_int4_repack(codes, iscales, N, K).reshape(-1))
    y2 = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def ref_int4(yh, x=x, codes=codes, iscales=iscales, N=N, K=K):
        rows = np.arange(0, N, 43)
        yr, ar = i4.qmm_int4(x, codes, iscales, N, K, rows=rows)
        return yh[:, rows], yr, ar
    out.append(("int4", lambda s, xd=xd, gi=gi, y=y2, M=M, N=N, K=K:
                sbb.qmm_run_int4(h, xd, gi, y, M, N, K, stream=s), y2, ref_int4))
    return out


def test_graph_replays_match_eager(h):
    calls = _calls(h)
    stream = torch.cuda.current_stream()
    for _, launch, y, _ in calls:
        launch(stream)
    torch.cuda.synchronize()
    eager = [y.clone() for _, _, y, _ in calls]
    for (label, _, _, ref), ye in zip(calls, eager):
        got, yr, ar = ref(ye.cpu().numpy().astype(np.float64))
        assert np.all(np.abs(got - yr) <= TOL * ar), label

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _, launch, _, _ in calls:  # warm the calls outside the capture
            launch(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for _, launch, _, _ in calls:
            launch(cap)
    torch.cuda.synchronize()

    for rep in range(4):
        for _, _, y, _ in calls:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (label, _, y, _), ye in zip(calls, eager):
            assert torch.equal(y.view(torch.int32), ye.view(torch.int32)), \
                "replay %d: %s differs from the eager result" % (rep, label)
        # eager work between replays: the same calls again, checked too
        for _, launch, _, _ in calls:
            launch(stream)
        torch.cuda.synchronize()
        for (label, _, y, _), ye in zip(calls, eager):
            assert torch.equal(y.view(torch.int32), ye.view(torch.int32)), \
                "eager run after replay %d: %s differs" % (rep, label)

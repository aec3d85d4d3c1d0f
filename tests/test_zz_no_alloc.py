"""The allocation-free entry point (qmm_run_static) against qmm_run.

Two calls in a row through the C ABI, the second with a smaller input, each
compared bitwise with qmm_run on a fresh handle (same launch plan, same
kernels) and with the oracle at the product's gate; both calls use split-K
across workgroups, so the static scratch (partial sums and arrival
counters) is what they run on. A plan too large for the scratch is refused
with QMM_ERR_SCRATCH and writes nothing. A seeded sequence of 60 small
ragged calls, most of them split-K, runs on the same scratch one after another,
and a captured HIP graph of such calls replays bitwise like the eager calls.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import skinny_bit_block_amd as sbb  # noqa: E402

pytestmark = pytest.mark.gpu

SEED = 20261202


def _case(M, N, K, tag):
    W = synth.weights(N, K, tensor=5000 + tag, seed=SEED)
    x = synth.acts(M, K, tensor=6000 + tag, seed=SEED)
    return x, W


def test_static_entry_matches_qmm_run_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = sbb.qmm_create(0)
    try:
        cases = [(16, 151936, 5120), (8, 5120, 17408)]  # the second is smaller
        for i, (M, N, K) in enumerate(cases):
            p = sbb.qmm_query_plan(h, M, N, K)
            assert p["workspace_bytes"] > 0, "the case must use split-K across workgroups"
            x, W = _case(M, N, K, i)
            xd = torch.from_numpy(x).cuda()
            Wd = torch.from_numpy(W.reshape(-1)).cuda()
            ys = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
            yr = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
            s = torch.cuda.current_stream().cuda_stream
            rc = sbb.qmm_run_static_raw(xd.data_ptr(), Wd.data_ptr(), ys.data_ptr(), M, N, K, s)
            assert rc == sbb.QMM_OK, sbb.qmm_status_string(rc)
            sbb.qmm_run(h, xd, Wd, yr, M, N, K)
            torch.cuda.synchronize()
            a = ys.cpu().numpy()
            b = yr.cpu().numpy()
            assert np.all(np.isfinite(a))
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "call %d differs" % i
            yref, aref = oracle.qmm(x, W, N, K)
            assert np.all(np.abs(a.astype(np.float64) - yref) <= 2e-3 * aref), "call %d" % i
    finally:
        sbb.qmm_destroy(h)


def test_static_entry_refuses_oversized_plans():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M, N, K = 32, 151936, 5120
    x = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    W = torch.zeros(sbb.qmm_weight_bytes(N, K), dtype=torch.uint8, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    rc = sbb.qmm_run_static_raw(x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K,
                                torch.cuda.current_stream().cuda_stream)
    assert rc == sbb.QMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_static_entry_seeded_sequence():
    # 60 calls in a row on small ragged matrices: their automatic plans split K
    # across workgroups heavily, so each call reuses the static partials and
    # the arrival counters the previous one left (which must be back at zero);
    # every call matches qmm_run bitwise and the oracle at the gate, and every
    # plan's loads are replayed on the host first
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import test_address_sim as addr
    rng = np.random.default_rng(20261206)
    h = sbb.qmm_create(0)
    s = torch.cuda.current_stream().cuda_stream
    split_k = 0
    try:
        for i in range(60):
            M = int(rng.integers(1, 33))
            N = int(rng.choice([1, 3, 16, 17, 33, 100, 257, 1000, 2047]))
            K = 256 * int(rng.integers(1, 18))
            p = sbb.qmm_query_plan(h, M, N, K)
            addr.replay(p, M, N, K)
            split_k += p["workspace_bytes"] > 0
            x, W = _case(M, N, K, 100 + i)
            xd = torch.from_numpy(x).cuda()
            Wd = torch.from_numpy(W.reshape(-1)).cuda()
            ys = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
            yr = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
            rc = sbb.qmm_run_static_raw(xd.data_ptr(), Wd.data_ptr(), ys.data_ptr(), M, N, K, s)
            assert rc == sbb.QMM_OK, (i, M, N, K, sbb.qmm_status_string(rc))
            sbb.qmm_run(h, xd, Wd, yr, M, N, K)
            torch.cuda.synchronize()
            a, b = ys.cpu().numpy(), yr.cpu().numpy()
            what = "call %d: M=%d N=%d K=%d" % (i, M, N, K)
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what
            yref, aref = oracle.qmm(x, W, N, K)
            assert np.all(np.abs(a.astype(np.float64) - yref) <= 2e-3 * aref), what
    finally:
        sbb.qmm_destroy(h)
    assert split_k >= 30  # most of the sequence runs on the static split-K scratch


def test_static_entry_in_a_graph():
    # the use the entry point is for: calls captured into a HIP graph. The
    # first call on the device (its set-up) is made before the capture, as a
    # warm-up; then the captured sequence is replayed four times with eager
    # calls on the same scratch and synchronizations in between, and every
    # replay must equal the eager results bitwise
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = [(8, 5120, 17408), (4, 1000, 2560), (1, 300, 4352), (32, 2047, 1280)]
    bufs = []
    for i, (M, N, K) in enumerate(cases):
        x, W = _case(M, N, K, 300 + i)
        bufs.append((M, N, K, torch.from_numpy(x).cuda(), torch.from_numpy(W.reshape(-1)).cuda(),
                     torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")))

    def run(stream, outs):
        for (M, N, K, xd, Wd, _), y in zip(bufs, outs):
            rc = sbb.qmm_run_static_raw(xd.data_ptr(), Wd.data_ptr(), y.data_ptr(), M, N, K, stream)
            assert rc == sbb.QMM_OK, sbb.qmm_status_string(rc)

    eager = [torch.full_like(b[5], np.nan) for b in bufs]
    run(torch.cuda.current_stream().cuda_stream, eager)  # warm-up and reference
    torch.cuda.synchronize()
    graph_out = [b[5] for b in bufs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        run(side.cuda_stream, graph_out)
    torch.cuda.synchronize()
    for rep in range(4):
        for y in graph_out:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(graph_out, eager)):
            assert torch.equal(y.view(torch.int32), e.view(torch.int32)), "replay %d, call %d" % (rep, i)
        again = [torch.full_like(e, np.nan) for e in eager]  # eager work on the same scratch
        run(torch.cuda.current_stream().cuda_stream, again)
        torch.cuda.synchronize()
        for i, (a, e) in enumerate(zip(again, eager)):
            assert torch.equal(a.view(torch.int32), e.view(torch.int32)), "eager %d, call %d" % (rep, i)

"""The allocation-free entry point (qmm_run_static) against qmm_run.

Two calls in a row through the C ABI, the second with a smaller input, each
compared bitwise with qmm_run on a fresh handle (same launch plan, same
kernels) and with the oracle at the product's gate; both calls use split-K
across workgroups, so the static scratch (partial sums and arrival
counters) is what they run on. A plan too large for the scratch is refused
with QMM_ERR_SCRATCH and writes nothing.
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

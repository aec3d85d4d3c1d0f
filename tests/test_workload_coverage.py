"""Every (matrix shape, row count) that the benchmark times has a GPU parity case."""
from skinny_bit_block_amd import accounting as acc

import workload_cases as wc


def test_every_pass_call_has_a_parity_case():
    missing = sorted({(N, K, M) for _, N, K in acc.full_pass_shapes() for M in wc.PASS_ROWS
                      if not wc.covered(N, K, M)})
    assert not missing, "pass calls without a GPU parity case: %s" % missing


def test_every_workload_config_has_a_parity_case():
    missing = [(N, K, M) for N, K, ms in wc.WORKLOADS for M in ms if not wc.covered(N, K, M)]
    assert not missing, "workload configs without a GPU parity case: %s" % missing


def test_parametrization_is_the_table():
    import test_gpu_parity as t
    names = {p[0] for p in wc.params()}
    assert names == set(wc.CASES)
    assert t.WORKLOAD_PARAMS == wc.params()


def test_every_fused_pass_call_has_a_parity_case():
    # the fused-projection pass calls each layer's five same-input 5120x5120
    # projections as one 25600-row matrix, the rest as in the full pass
    shapes = {(5 * N, K) if N == K else (N, K) for _, N, K in acc.full_pass_shapes()} | {(5120, 5120)}
    missing = sorted((N, K, M) for N, K in shapes for M in wc.PASS_ROWS if not wc.covered(N, K, M))
    assert not missing, "fused-pass calls without a GPU parity case: %s" % missing

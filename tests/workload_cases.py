"""Row counts at which the GPU parity tests run each workload shape.

One table drives both the GPU parametrization (tests/test_gpu_parity.py) and
the CPU check that every (shape, rows) pair the benchmark runs has a parity
case (tests/test_workload_coverage.py). Every case compares the whole output
with the oracle, at the launch plan the library picks for that call (the plan
the benchmark times).
"""

# (N, K, row counts, activation scale)
CASES = {
    "single_2048": (2048, 2048, [1, 4, 16], 1.0),
    "square_5120": (5120, 5120, [1, 2, 4, 8, 16, 32], 1.0),
    "gate_up": (34816, 5120, [1, 2, 4, 7, 8, 9, 16, 32], 1.0),
    "down": (5120, 17408, [1, 4, 6, 8, 12, 16, 32], 0.1),
    "lm_head": (151936, 5120, [1, 4, 7, 8, 16, 32], 1.0),
    # each layer's five same-input projections as one call (the fused-projection pass)
    "fused_5x5120": (25600, 5120, [1, 4, 8, 16, 32], 1.0),
}

# rows of the timed full pass (the headline passes and the 32-row pass)
PASS_ROWS = (1, 4, 8, 16, 32)

# the single-matrix workloads: (N, K, row counts)
WORKLOADS = [
    (2048, 2048, [4]),
    (34816, 5120, [1, 2, 4, 7, 8, 9, 16]),
    (5120, 17408, [1, 4, 8, 16]),
    (151936, 5120, [1, 7]),
]


def params():
    """[(name, N, K, M, xscale)] for pytest parametrization."""
    out = []
    for name, (N, K, ms, xs) in CASES.items():
        for M in ms:
            out.append((name, N, K, M, xs))
    return out


def covered(N, K, M):
    return any(n == N and k == K and M in ms for n, k, ms, _ in CASES.values())

"""Every global load of the kernels stays inside W and x: a host replay of the
kernels' load-address arithmetic for every launch plan the library makes.

The replay restates, in numpy, the index math of the weight stream (the
per-lane chunk offsets of a stage, the partial last stage whose chunks past
the slice end step back to the slice's last block, the first stage of a wave
with no work, the ragged last row tile whose missing rows re-read its last
row), the split of K among workgroups and waves (make_split) and the
activation staging loads (the chunked unit walk of the x lead, with the
kernel's float-reciprocal division and its clamp for lanes past the last
unit). Plans come from the library's own planner (planning-only handle):
every launch-table entry at every row count for the three weight formats and
for expert-indexed calls, the forced launch shapes the GPU tests run, and a
seeded sweep of forced shapes over ragged small matrices. Grids are replayed
both as planned and as persistent grids of a few workgroups.

The index math is restated here, not shared: a change to the kernels' load
arithmetic must be mirrored in this file, which then checks it again.
"""
import numpy as np
import pytest

import skinny_bit_block_amd as sbb

BLOCK_BYTES = 144           # one super-block (or one 144-byte group of the other formats)
STAGE_BLOCKS = 4            # super-blocks per stage of a wave
SEG_CHUNKS = 9 * STAGE_BLOCKS   # 16-byte chunks per row segment of a stage
STAGE_LOADS = 16 * SEG_CHUNKS // 64
VECTOR_LEAD, TILED_LEAD = 8, 16  # x units per thread per chunk of the x lead


# ------------------------------------------------------------------ weight stream

def stage_lane(nb, rows):
    """Per-lane chunk offsets of a stage: (goff[64, 9], blk[64, 9])."""
    q = np.arange(64)[:, None] + 64 * np.arange(STAGE_LOADS)[None, :]
    row, cc = q // SEG_CHUNKS, q % SEG_CHUNKS
    rr = np.minimum(row, rows - 1)
    goff = (rr * nb * BLOCK_BYTES + cc * 16).astype(np.int64)
    assert goff.max() < 2 ** 32  # a uint32 in the kernel
    return goff, cc // 9


def stage_offsets(goff, blk, s, nbw):
    """Byte offsets from the stage's tile-row base of the 16-byte loads of stage s."""
    sbase = s * STAGE_BLOCKS * BLOCK_BYTES
    if (s + 1) * STAGE_BLOCKS <= nbw:
        return sbase + goff
    last = nbw - 1 - s * STAGE_BLOCKS
    back = np.where(blk > last, (blk - last) * BLOCK_BYTES, 0)
    return sbase + ((goff - back) & 0xFFFFFFFF)  # 32-bit arithmetic in the kernel


def make_split(bx, by, wave, waves, wsplit, nbs, nb, ntiles, grid_x):
    wslice, wtile, T = wave % wsplit, wave // wsplit, waves // wsplit
    kb0_wg = by * wsplit * nbs
    nbw_wg = min(wsplit * nbs, nb - kb0_wg)
    kb0 = kb0_wg + wslice * nbs
    nbw = max(0, min(nbs, nb - kb0))
    first_wg, step = bx * T, grid_x * T
    iters = (ntiles - 1 - first_wg) // step + 1 if first_wg < ntiles else 0
    return dict(wtile=wtile, T=T, kb0_wg=kb0_wg, nbw_wg=nbw_wg, kb0=kb0, nbw=nbw, step=step,
                iters=iters)


def wave_walk(c, bx, ntiles, nstages):
    """(tile, stage) pairs a wave loads, replayed step by step the way the kernel's
    flat loop runs (first stage, then one prefetch per step)."""
    tile = bx * c["T"] + c["wtile"]
    loads = []
    if tile < ntiles and nstages > 0:
        loads.append((tile, 0))
    ns = max(nstages, 1)
    cs = 0
    for _ in range(c["iters"] * ns):
        if tile < ntiles and nstages > 0:
            nt, nsn = tile, cs + 1
            if nsn == nstages:
                nsn, nt = 0, nt + c["step"]
            if nt < ntiles:
                loads.append((nt, nsn))
        cs += 1
        if cs == ns:
            cs = 0
            tile += c["step"]
    return loads


def check_weights(p, N, K, grid_x, walk_limit=400):
    """Bounds of every weight load of a plan at grid_x workgroups per slice
    range. Per wave the loaded tiles are an arithmetic progression (checked
    step by step against the kernel's loop for the first and last workgroup)
    and a tile's loads differ from another's only by the tile's base and, for
    the ragged last tile, its row count, so the extremes of each wave's walk
    bound all of its loads; every (K slice, tile) must be walked once."""
    nb, ntiles = K // 256, (N + 15) // 16
    waves, wsplit, nbs = p["waves_per_wg"], p["wave_splits"], p["blocks_per_split"]
    grid_y = (p["splits"] + wsplit - 1) // wsplit
    row_bytes, total = nb * BLOCK_BYTES, N * nb * BLOCK_BYTES
    rows_last = N - 16 * (ntiles - 1)
    offs = {}

    def stage_range(rows, s, nbw):
        key = (rows, s, nbw)
        if key not in offs:
            o = stage_offsets(*stage_lane(nb, rows), s, nbw)
            offs[key] = (int(o.min()), int(o.max()))
        return offs[key]

    bxs = np.arange(grid_x, dtype=np.int64)
    for by in range(grid_y):
        for wave in range(waves):
            c = make_split(0, by, wave, waves, wsplit, nbs, nb, ntiles, grid_x)
            assert c["nbw_wg"] >= 1 and c["nbw"] <= nbs
            nstages = (c["nbw"] + STAGE_BLOCKS - 1) // STAGE_BLOCKS
            T, step = c["T"], c["step"]
            tile0 = bxs * T + c["wtile"]
            first_wg = bxs * T
            iters = np.where(first_wg < ntiles, (ntiles - 1 - first_wg) // step + 1, 0)
            # the replayed loop agrees with the closed form for the end workgroups
            for bx in sorted({0, grid_x - 1}):
                cb = make_split(bx, by, wave, waves, wsplit, nbs, nb, ntiles, grid_x)
                assert cb["iters"] == iters[bx]
                if cb["iters"] * max(nstages, 1) <= walk_limit:
                    loads = wave_walk(cb, bx, ntiles, nstages)
                    k = np.arange(cb["iters"])
                    want = [t for t in (bx * T + c["wtile"] + step * k) if t < ntiles] if nstages else []
                    assert loads == [(int(t), s) for t in want for s in range(nstages)]
            if not ((tile0 < ntiles) & (nstages > 0)).all():
                # first stage of a wave without work: the matrix's first rows
                lo, hi = stage_range(min(16, N), 0, nb)
                assert lo >= 0 and hi + 16 <= total
            if nstages == 0:
                continue
            has = tile0 < ntiles
            kl = np.minimum(iters - 1, (ntiles - 1 - tile0) // step)
            first, last = tile0[has], (tile0 + step * kl)[has]
            slice_base = c["kb0"] * BLOCK_BYTES
            own = min(c["nbw"], nb - c["kb0"]) * BLOCK_BYTES
            if not has.any():
                continue
            for s in range(nstages):
                lo_f, _ = stage_range(16 if ntiles > 1 else rows_last, s, c["nbw"])
                assert lo_f >= 0 and slice_base + int(first.min()) * 16 * row_bytes + lo_f >= 0
                for rl, sel in ((16, last < ntiles - 1), (rows_last, last == ntiles - 1)):
                    if not sel.any():
                        continue
                    lo2, hi2 = stage_range(rl, s, c["nbw"])
                    end = slice_base + int(last[sel].max()) * 16 * row_bytes + hi2 + 16
                    assert end <= total, (p, N, K, grid_x, by, wave, s, end, total)
                    # the stage stays inside its own tile's rows and K slice
                    assert lo2 >= 0 and hi2 + 16 <= (rl - 1) * row_bytes + own
    # each (K slice, tile) is walked by exactly one wave
    for by in range(grid_y):
        for ws in range(wsplit):
            if by * wsplit * nbs + ws * nbs >= nb:
                continue
            seen = np.zeros(ntiles, dtype=np.int64)
            for wt in range(waves // wsplit):
                tile0 = bxs * (waves // wsplit) + wt
                kmax = (ntiles - 1) // (grid_x * (waves // wsplit)) + 1
                t = (tile0[:, None] + grid_x * (waves // wsplit) * np.arange(kmax)[None, :]).ravel()
                np.add.at(seen, t[t < ntiles], 1)
            assert (seen == 1).all(), (p, N, K, grid_x, by, ws)


# ------------------------------------------------------------------ activations

def div_small(u, d, rcp):
    q = (u.astype(np.float32) * rcp).astype(np.int64)
    rem = u - q * d
    return q + np.where(rem < 0, -1, np.where(rem >= d, 1, 0))


def check_x(p, M, K, lead):
    """Bounds of every activation load of the x lead of each slice range."""
    nb = K // 256
    waves, wsplit, nbs = p["waves_per_wg"], p["wave_splits"], p["blocks_per_split"]
    grid_y = (p["splits"] + wsplit - 1) // wsplit
    nthr = 64 * waves
    tid = np.arange(nthr, dtype=np.int64)
    t, g = tid & 7, (tid >> 3) & 3
    rcp = np.float32(1.0) / np.float32(M)
    xfloats = M * K
    for by in range(grid_y):
        kb0_wg = by * wsplit * nbs
        nbw_wg = min(wsplit * nbs, nb - kb0_wg)
        units = M * nbw_wg * 32
        last = units - 1
        c0 = kb0_wg * 256 + 64 * g + 4 * t
        clamp = (M - 1) * K + (nbw_wg - 1) * 256 + c0
        left = (units + nthr - 1) // nthr
        base, chunks = 0, []
        while left > lead:
            chunks.append((base, lead))
            left -= lead
            base += lead * nthr
        chunks.append((base, left))
        covered = np.zeros(units, dtype=np.int64)
        for base, nu in chunks:
            rest = (base + tid) >> 5
            bl = div_small(rest, M, rcp)
            s = nthr >> 5
            dq = int(div_small(np.array([s]), M, rcp)[0])
            m, dr = rest - bl * M, s - dq * M
            for j in range(nu):
                u = base + j * nthr + tid
                real = u <= last
                # the walk's (row, block) is the unit's own
                assert (m[real] == (u[real] >> 5) % M).all() and (bl[real] == (u[real] >> 5) // M).all()
                off = np.where(real, m * K + (bl << 8) + c0, clamp)
                assert off.min() >= 0 and off.max() < 2 ** 32
                assert (off + 32 + 4).max() <= xfloats  # both 16-byte loads of the unit
                covered[u[real]] += 1
                m, bl = m + dr, bl + dq
                wrap = m >= M
                m, bl = np.where(wrap, m - M, m), np.where(wrap, bl + 1, bl)
        assert (covered == 1).all()  # every unit of the range is loaded once


# ------------------------------------------------------------------ plans

@pytest.fixture(scope="module")
def planner():
    h = sbb.qmm_create(sbb.QMM_DEVICE_NONE)
    yield h
    sbb.qmm_destroy(h)


def plan(h, fmt, slots, M, N, K, kernel=sbb.KERNEL_AUTO, shape=(0, 0, 0), wsplit=0):
    sbb.qmm_set_kernel(h, kernel)
    sbb.qmm_set_shape(h, *shape)
    sbb.qmm_set_wave_splits(h, wsplit)
    try:
        return sbb.qmm_query_plan_format(h, fmt, slots, M, N, K)
    except sbb.QmmError as e:
        assert e.status in (sbb.QMM_ERR_INVALID_ARG, sbb.QMM_ERR_SHAPE)
        return None
    finally:
        sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)
        sbb.qmm_set_shape(h, 0, 0, 0)
        sbb.qmm_set_wave_splits(h, 0)


def replay(p, M, N, K, grids=()):
    lead = TILED_LEAD if p["kernel"] == sbb.KERNEL_TILED else VECTOR_LEAD
    check_x(p, M, K, lead)
    check_weights(p, N, K, p["grid_x"])
    for gx in grids:  # persistent grids: fewer workgroups walk more tiles
        if gx < p["grid_x"]:
            check_weights(p, N, K, gx)


TABLE_SHAPES = [(5120, 5120), (34816, 5120), (5120, 17408), (151936, 5120), (2048, 2048),
                (25600, 5120)]


@pytest.mark.parametrize("fmt", [sbb.FORMAT_KQUANT, sbb.FORMAT_NVFP4, sbb.FORMAT_INT4])
def test_table_plans(planner, fmt):
    # every launch-table entry at every row count, as planned and as persistent
    # grids (the device caps the grid at its residency)
    for N, K in TABLE_SHAPES:
        for M in range(1, 33):
            p = plan(planner, fmt, 0, M, N, K)
            assert p is not None, (fmt, M, N, K)
            replay(p, M, N, K, grids=(1, 7, 256))


def test_expert_plans(planner):
    # expert-indexed calls: each slot streams one expert's matrix with the rows
    # that use it (its own row count, at most the call's)
    for N, K in [(34816, 5120), (300, 1280), (1000, 2560), (700, 1536)]:
        for M in (1, 3, 8, 12, 17, 32):
            for slots in sorted({1, min(M, 4), min(M, 8)}):
                p = plan(planner, sbb.FORMAT_KQUANT, slots, M, N, K)
                assert p is not None
                for m in sorted({1, M}):
                    replay(p, m, N, K, grids=(1, 5))


GPU_TEST_SHAPES = [((1, 1, 0), 0), ((2, 3, 0), 0), ((4, 2, 0), 0), ((8, 5, 0), 0), ((8, 1, 0), 0),
                   ((1, 10, 0), 0), ((4, 7, 500), 0), ((8, 4, 63), 0), ((1, 1, 1), 0), ((2, 3, 5), 0),
                   ((4, 1, 3), 0), ((8, 2, 1), 0), ((4, 10, 2), 0),
                   ((2, 2, 0), 2), ((4, 4, 0), 4), ((5, 5, 0), 5), ((4, 8, 0), 4), ((8, 4, 0), 4),
                   ((6, 3, 0), 3), ((8, 8, 3), 2), ((4, 10, 1), 2), ((3, 3, 2), 3), ((8, 10, 0), 8),
                   ((7, 7, 0), 7), ((2, 10, 0), 2), ((4, 10, 0), 4),
                   ((4, 3, 0), 0), ((4, 2, 2), 2), ((2, 1, 1), 0), ((8, 5, 0), 0),
                   ((4, 1, 0), 1), ((8, 2, 0), 1), ((4, 5, 1), 1), ((4, 2, 0), 2), ((8, 10, 3), 2),
                   ((2, 3, 1), 1), ((6, 2, 0), 2), ((3, 1, 0), 1)]


def test_forced_shapes_of_the_gpu_tests(planner):
    n = 0
    for shape, wsplit in GPU_TEST_SHAPES:
        for M in (1, 3, 5, 7, 8, 12, 16, 20, 32):
            for kernel in (sbb.KERNEL_VECTOR, sbb.KERNEL_TILED):
                for fmt in ((0, 1, 2) if kernel == sbb.KERNEL_TILED else (0,)):
                    p = plan(planner, fmt, 0, M, 1000, 2560, kernel, shape, wsplit)
                    if p is not None:
                        replay(p, M, 1000, 2560)
                        n += 1
    assert n > 500


def test_seeded_sweep_of_ragged_shapes(planner):
    # forced shapes over ragged matrices: 1..3 row tiles and a partial one,
    # K of 1..17 super-blocks (partial last stages of every length)
    rng = np.random.default_rng(20261202)
    Ns = [1, 3, 15, 16, 17, 33, 129, 300, 333, 1000, 2047]
    Ks = [256 * b for b in (1, 2, 3, 4, 5, 6, 7, 9, 10, 13, 17)]
    n = 0
    while n < 1200:
        N, K = int(rng.choice(Ns)), int(rng.choice(Ks))
        M = int(rng.integers(1, 33))
        kernel = int(rng.choice([sbb.KERNEL_VECTOR, sbb.KERNEL_TILED]))
        fmt = int(rng.choice([0, 1, 2])) if kernel == sbb.KERNEL_TILED else 0
        waves = int(rng.integers(1, 9))
        shape = (waves, int(rng.integers(0, K // 256 + 1)), int(rng.choice([0, 0, 1, 2, 3, 7])))
        wsplit = int(rng.choice([0, 1, 1, 2, 3, 4, 8]))
        p = plan(planner, fmt, 0, M, N, K, kernel, shape, wsplit)
        if p is None:
            continue
        replay(p, M, N, K)
        n += 1


# (N, K, row counts): x of the longest rows stays under 0.5 GB
LONG_K = [(1, 1 << 24, (1, 7)), (17, 1 << 22, (1, 7)), (20, 1 << 20, (1, 7, 32)),
          (5, 1 << 19, (1, 7, 32)), (33, 1 << 18, (1, 7, 32))]


def test_long_k_plans(planner):
    # K far beyond the workloads' (up to the largest the library takes, 2^24):
    # many K slices over few row tiles, long 32-bit in-wave offsets; both
    # kernels, at the row counts the GPU test runs
    for N, K, Ms in LONG_K:
        for M, kernel in ((1, sbb.KERNEL_AUTO), (1, sbb.KERNEL_TILED), (7, sbb.KERNEL_AUTO),
                          (7, sbb.KERNEL_VECTOR), (32, sbb.KERNEL_AUTO)):
            if M not in Ms:
                continue
            p = plan(planner, sbb.FORMAT_KQUANT, 0, M, N, K, kernel)
            assert p is not None, (M, N, K, kernel)
            replay(p, M, N, K, grids=(1,))


# the other weight formats' long-K GPU cases (M, N, K)
LONG_K_FORMATS = [(1, 1, 1 << 22), (7, 5, 1 << 20), (32, 3, 1 << 18)]


@pytest.mark.parametrize("fmt", [sbb.FORMAT_NVFP4, sbb.FORMAT_INT4])
def test_long_k_plans_of_the_group_formats(planner, fmt):
    for M, N, K in LONG_K_FORMATS:
        p = plan(planner, fmt, 0, M, N, K)
        assert p is not None, (fmt, M, N, K)
        replay(p, M, N, K, grids=(1,))


def test_long_k_expert_plans(planner):
    # the expert-indexed long-K GPU cases: each slot streams one expert with
    # the rows that use it
    for M, E, N, K in [(7, 4, 5, 1 << 20), (32, 3, 3, 1 << 18), (2, 2, 17, 1 << 19)]:
        for slots in sorted({1, min(M, E)}):
            p = plan(planner, sbb.FORMAT_KQUANT, slots, M, N, K)
            assert p is not None, (M, E, N, K, slots)
            for m in sorted({1, M}):
                replay(p, m, N, K, grids=(1,))


def test_replay_catches_a_stage_past_the_slice_end():
    # the replay flags the fault class it guards: a partial stage whose clamp
    # starts from a stage wholly past the slice end wraps the 32-bit offset
    goff, blk = stage_lane(20, 16)
    o = stage_offsets(goff, blk, 5, 20)  # stage 5 of a 20-block slice: past the end
    assert o.max() >= 2 ** 32 - 4 * BLOCK_BYTES
    ok = stage_offsets(goff, blk, 4, 19)  # stage 4 of 19 blocks: 3 real, 1 stepped back
    assert ok.max() + 16 <= 15 * 20 * BLOCK_BYTES + 19 * BLOCK_BYTES

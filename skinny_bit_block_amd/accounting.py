"""Byte-exact accounting of the weight stream and the roofline guard.

Weight bytes of an N x K matrix in 144-byte / 256-weight super-blocks are
144 * N * K / 256 (4.5 bits per weight); GB = 1e9 bytes. This is the
weight-only convention of the pages: FlashRT issue #153 (the Thor NVFP4 decode
page) quotes "effective weight bandwidth" for lm_head and gate+up at M = 1 and
M = 7 exactly this way, and "sixi-asi 0.9", section "The patch", derives the
~58 ms floor of a pass from 15.8 GB at 273 GB/s. The same section's rule is
kept literally: a time shorter than the bytes need at peak bandwidth is a bug
report, so `check_roofline` raises.
"""

BLOCK_WEIGHTS = 256
BLOCK_BYTES = 144
HBM_PEAK_BYTES_PER_S = 8.0e12  # MI355X HBM3E, AMD's published figure


class RooflineViolation(RuntimeError):
    """A measured time beats the memory roofline: the measurement is wrong."""


def weight_bytes(N, K):
    if K % BLOCK_WEIGHTS or N < 0 or K < 0:
        raise ValueError("K must be a multiple of 256")
    return int(N) * (int(K) // BLOCK_WEIGHTS) * BLOCK_BYTES


def call_bytes(M, N, K):
    """Algorithmic HBM bytes of one call: weights + fp32 x + fp32 y."""
    return weight_bytes(N, K) + 4 * int(M) * int(K) + 4 * int(M) * int(N)


def call_flops(M, N, K):
    return 2 * int(M) * int(N) * int(K)


def gbs(nbytes, seconds):
    return nbytes / seconds / 1e9


def pct_of(nbytes, seconds, peak_bytes_per_s):
    return 100.0 * nbytes / seconds / peak_bytes_per_s


def floor_seconds(nbytes, peak_bytes_per_s=HBM_PEAK_BYTES_PER_S):
    return nbytes / peak_bytes_per_s


def check_roofline(nbytes, seconds, peak_bytes_per_s=HBM_PEAK_BYTES_PER_S, what="call"):
    """Raise RooflineViolation if `seconds` is shorter than reading `nbytes` at peak."""
    floor = floor_seconds(nbytes, peak_bytes_per_s)
    if seconds < floor:
        raise RooflineViolation(
            "%s: %.3f us is below the %.3f us it takes to read %d bytes at %.1f GB/s"
            % (what, seconds * 1e6, floor * 1e6, nbytes, peak_bytes_per_s / 1e9))
    return floor


def check_counter_bytes(counter_bytes, nbytes, frac=0.98, what="call"):
    """Raise if the memory counters saw fewer bytes than the weights: a cache served them."""
    if counter_bytes < frac * nbytes:
        raise RooflineViolation("%s: counters read %d bytes, fewer than %.2f x %d weight bytes"
                                % (what, counter_bytes, frac, nbytes))


# The full verify pass of the pages' 27B hybrid model, as synthetic shapes:
# 64 layers of six 5120 x 5120 projections, the fused gate+up (2 x 17408 rows,
# K = 5120) and the down projection (K = 17408), plus a 151936-row lm_head;
# 15,725,813,760 weight bytes, the ~15.8 GB per pass of "sixi-asi 0.11",
# section "Why sixteen streams were the ceiling". The six square matrices per
# layer are a reading (q, k, v, o and two more of the same class); four give
# only 13.84 GB.
LAYERS = 64
SQUARE_PER_LAYER = 6
HIDDEN = 5120
FFN = 17408
VOCAB = 151936


def full_pass_shapes():
    """[(name, N, K)] in launch order for one pass."""
    shapes = []
    for layer in range(LAYERS):
        for i in range(SQUARE_PER_LAYER):
            shapes.append(("L%d.proj%d" % (layer, i), HIDDEN, HIDDEN))
        shapes.append(("L%d.gate_up" % layer, 2 * FFN, HIDDEN))
        shapes.append(("L%d.down" % layer, HIDDEN, FFN))
    shapes.append(("lm_head", VOCAB, HIDDEN))
    return shapes


def full_pass_weight_bytes():
    return sum(weight_bytes(N, K) for _, N, K in full_pass_shapes())

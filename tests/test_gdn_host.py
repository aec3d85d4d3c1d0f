"""The recurrent-update entry point's host-side checks (no GPU needed: every
error is found before the launch, and fake pointers are never dereferenced)."""
import pytest

import skinny_bit_block_amd as sbb
from skinny_bit_block_amd import gdn

B, M, H, L, D = 2, 3, 4, 5, 128
BASE = 1 << 32
STATE = BASE                                # B*H*D*D*4 = 512 KiB
LOG = BASE + (1 << 24)                      # log arrays, 1 MiB apart
NEW = BASE + (1 << 26)                      # new-row arrays, 1 MiB apart
OUT = BASE + (1 << 28)


def args(**over):
    a = dict(state=STATE, k_log=LOG, v_log=LOG + (1 << 20), gate_log=LOG + (2 << 20),
             beta_log=LOG + (3 << 20), n_log=LOG + (4 << 20), L=L, q=NEW, k=NEW + (1 << 20),
             v=NEW + (2 << 20), gate=NEW + (3 << 20), beta=NEW + (4 << 20), commit=NEW + (5 << 20),
             o=OUT, B=B, M=M, H=H, dk=D, dv=D)
    a.update(over)
    return a


def call(**over):
    a = args(**over)
    return gdn.gdn_replay_update_raw(a["state"], a["k_log"], a["v_log"], a["gate_log"], a["beta_log"],
                                     a["n_log"], a["L"], a["q"], a["k"], a["v"], a["gate"], a["beta"],
                                     a["commit"], a["o"], a["B"], a["M"], a["H"], a["dk"], a["dv"])


def test_valid_arguments_reach_the_device_query():
    # everything checks out; without a GPU the call stops at the device
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call() == sbb.QMM_ERR_NO_DEVICE
    # optional arrays: no log, no new rows, no commit
    assert call(L=0, k_log=None, v_log=None, gate_log=None, beta_log=None, n_log=None) == sbb.QMM_ERR_NO_DEVICE
    assert call(M=0, q=None, k=None, v=None, gate=None, beta=None, o=None) == sbb.QMM_ERR_NO_DEVICE
    assert call(commit=None) == sbb.QMM_ERR_NO_DEVICE


@pytest.mark.parametrize("over,status", [
    (dict(state=None), sbb.QMM_ERR_INVALID_ARG),
    (dict(B=0), sbb.QMM_ERR_INVALID_ARG),
    (dict(H=0), sbb.QMM_ERR_INVALID_ARG),
    (dict(M=-1), sbb.QMM_ERR_INVALID_ARG),
    (dict(L=-1), sbb.QMM_ERR_INVALID_ARG),
    (dict(dk=64), sbb.QMM_ERR_SHAPE),
    (dict(dv=256), sbb.QMM_ERR_SHAPE),
    (dict(k_log=None), sbb.QMM_ERR_INVALID_ARG),
    (dict(n_log=None), sbb.QMM_ERR_INVALID_ARG),
    (dict(q=None), sbb.QMM_ERR_INVALID_ARG),
    (dict(o=None), sbb.QMM_ERR_INVALID_ARG),
    (dict(B=1 << 30, H=8), sbb.QMM_ERR_INVALID_ARG),  # more than 2^31 - 1 workgroups
    (dict(B=1 << 20, H=16, L=(1 << 20) + 1), sbb.QMM_ERR_INVALID_ARG),  # over 2^40 log rows
    (dict(B=1 << 20, H=16, M=(1 << 20) + 1), sbb.QMM_ERR_INVALID_ARG),  # over 2^40 new rows
    (dict(B=(1 << 30) - 1, H=2, L=(1 << 31) - 1), sbb.QMM_ERR_INVALID_ARG),  # byte counts past 2^64
    (dict(state=STATE + 2), sbb.QMM_ERR_ALIGN),
    (dict(gate=NEW + (3 << 20) + 1), sbb.QMM_ERR_ALIGN),
    (dict(o=STATE + 4096), sbb.QMM_ERR_OVERLAP),               # o inside the state
    (dict(k=STATE + B * H * D * D * 4 - 4), sbb.QMM_ERR_OVERLAP),  # an input over the state's end
    (dict(o=NEW + (2 << 20) + 8), sbb.QMM_ERR_OVERLAP),        # o over v
    (dict(commit=OUT + 4), sbb.QMM_ERR_OVERLAP),               # commit under o
])
def test_argument_errors(over, status):
    assert call(**over) == status


def test_call_bytes():
    # 32 sequences x 48 heads of 128 x 128 fp32: 3 MiB of state each, read,
    # and written for the committing ones; rows: k, v, gate, beta (+ q for new)
    st = 32 * 48 * 128 * 128 * 4
    assert st == 32 * 3 * 2 ** 20
    got = gdn.gdn_call_bytes(32, 4, 48, 128, 128, 100, 10)
    want = st + 10 * 48 * 128 * 128 * 4 + 100 * 48 * (128 + 128 + 2) * 4 + \
        32 * 4 * 48 * (2 * 128 + 128 + 2) * 4 + 32 * 4 * 48 * 128 * 4
    assert got == want
    assert gdn.gdn_call_bytes(-1, 4, 48, 128, 128, 0, 0) == 0


# ------------------------------------------------- overlap rule, property-based

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

NAMES = ["state", "k_log", "v_log", "gate_log", "beta_log", "n_log", "q", "k", "v", "gate", "beta",
         "commit", "o"]
INPUTS = NAMES[1:12]


def extents(Bn, Hn, Ln, Mn, with_commit):
    """Bytes of every array of a call, as the header documents them."""
    lrow, nrow = Bn * Ln * Hn, Bn * Mn * Hn
    e = {"state": Bn * Hn * D * D * 4, "k_log": lrow * D * 4, "v_log": lrow * D * 4,
         "gate_log": lrow * 4, "beta_log": lrow * 4, "n_log": Bn * 4 if Ln else 0,
         "q": nrow * D * 4, "k": nrow * D * 4, "v": nrow * D * 4, "gate": nrow * 4,
         "beta": nrow * 4, "commit": Bn * 4 if with_commit else 0, "o": nrow * D * 4}
    return e


def meets(a, na, b, nb):
    return na > 0 and nb > 0 and a < b + nb and b < a + na


@settings(max_examples=600, deadline=None, derandomize=True)
@given(data=st.data())
def test_overlap_rule(data):
    # arrays placed at random, often on top of one another: the call reports
    # QMM_ERR_ALIGN for a misaligned pointer, else QMM_ERR_OVERLAP exactly when
    # the state meets any other array or o meets an input, else it reaches the
    # device query (inputs may share memory with one another)
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: disjoint arrays would reach a launch")
    Bn, Hn = data.draw(st.integers(1, 3)), data.draw(st.integers(1, 3))
    Ln, Mn = data.draw(st.integers(0, 3)), data.draw(st.integers(0, 3))
    with_commit = data.draw(st.booleans())
    ext = extents(Bn, Hn, Ln, Mn, with_commit)
    used = [n for n in NAMES if ext[n] > 0]
    slots = data.draw(st.lists(st.integers(0, 11), min_size=len(used), max_size=len(used)))
    offs = data.draw(st.lists(st.integers(0, 1 << 17), min_size=len(used), max_size=len(used)))
    misalign = data.draw(st.sampled_from(used)) if data.draw(st.integers(0, 9)) == 0 else None
    ptr = {n: None for n in NAMES}
    for n, s, o in zip(used, slots, offs):
        ptr[n] = BASE + s * (1 << 22) + 4 * o + (2 if n == misalign else 0)
    a = dict(state=ptr["state"], L=Ln, B=Bn, M=Mn, H=Hn, dk=D, dv=D,
             **{n: ptr[n] for n in NAMES[1:]})
    got = call(**a)
    if misalign is not None:
        assert got == sbb.QMM_ERR_ALIGN, (a, got)
        hypothesis.event("misaligned")
        return
    clash = any(meets(ptr["state"], ext["state"], ptr[n], ext[n]) for n in NAMES[1:] if ptr[n]) or \
        any(meets(ptr["o"], ext["o"], ptr[n], ext[n]) for n in INPUTS if ptr[n] and ptr["o"])
    hypothesis.event("overlap" if clash else "disjoint")
    assert got == (sbb.QMM_ERR_OVERLAP if clash else sbb.QMM_ERR_NO_DEVICE), (a, got, clash)

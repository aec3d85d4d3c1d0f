"""The rocprofv3 summary tool on synthetic CSVs, and the counter guard applied
to the committed counter summary."""
import csv
import json
import os
import re

import pytest

from skinny_bit_block_amd import accounting as acc
from skinny_bit_block_amd import profile_summary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPES = {"square": (5120, 5120), "gate_up": (34816, 5120), "down": (5120, 17408),
          "lm_head": (151936, 5120), "single_2048": (2048, 2048)}


def _seq():
    launches = []
    for M in (1, 4):
        sym = "qmm_vector_kernel<1>" if M == 1 else "qmm_tiled_kernel<1, false, 0>"
        for shape in ("square", "square", "gate_up", "down", "lm_head"):
            N, K = SHAPES[shape]
            launches.append({"symbol": sym, "shape": shape, "M": M, "N": N, "K": K})
    launches.append({"symbol": "qmm_tiled_kernel<1, false, 0>", "shape": "config single_2048",
                     "M": 4, "N": 2048, "K": 2048})
    return {"kernel_source_sha256": "0123456789abcdef", "launches": launches}


def _write_trace(path, seq):
    cols = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        did, t = 1, 1000
        for i, s in enumerate(seq["launches"]):
            # a foreign kernel between the library's dispatches is ignored
            w.writerow(["KERNEL_DISPATCH", did, "void qmm::zero_u32(unsigned int*, int)", t, t + 500])
            did += 1
            us = acc.weight_bytes(s["N"], s["K"]) / 4e3  # 4 TB/s
            w.writerow(["KERNEL_DISPATCH", did, "void qmm::%s(qmm::Args)" % s["symbol"],
                        t, t + int(us * 1000)])
            did += 1
            t += 10 ** 6


def _write_counter(path, seq, name, scale, copy_kib=None):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        did = 7
        if copy_kib is not None:
            for _ in range(3):
                w.writerow([did, "__amd_rocclr_copyBuffer", name, copy_kib])
                did += 1
            return
        for s in seq["launches"]:
            b = acc.weight_bytes(s["N"], s["K"]) if name == "FETCH_SIZE" else 4 * s["M"] * s["N"]
            # two counter instances per dispatch (summed by the tool)
            w.writerow([did, "void qmm::%s(qmm::Args)" % s["symbol"], name, b / 1024.0 / scale / 2])
            w.writerow([did, "void qmm::%s(qmm::Args)" % s["symbol"], name, b / 1024.0 / scale / 2])
            did += 3


def test_trace_summary(tmp_path):
    seq = _seq()
    json.dump(seq, open(tmp_path / "seq.json", "w"))
    _write_trace(tmp_path / "t.csv", seq)
    ps.main(["trace", "--csv", str(tmp_path / "t.csv"), "--seq", str(tmp_path / "seq.json"),
             "--command", "cmd", "--out", str(tmp_path / "t.md")])
    text = open(tmp_path / "t.md").read()
    assert "kernel_source_sha256: 0123456789abcdef" in text
    means = dict(re.findall(r"mean_kernel_us\[(.+?)\]: ([\d.]+)", text))
    # the config launch is not part of the kernel's full-pass mean
    tiled = [acc.weight_bytes(*SHAPES[s]) / 4e3 for s in ("square", "square", "gate_up", "down", "lm_head")]
    assert float(means["qmm_tiled_kernel<1, false, 0>"]) == pytest.approx(sum(tiled) / 5, abs=2e-3)
    assert "| config single_2048 M=4 | 1 |" in text
    assert "| square M=1 | 2 |" in text


def test_trace_summary_rejects_a_mismatch(tmp_path):
    seq = _seq()
    _write_trace(tmp_path / "t.csv", seq)
    seq["launches"][3]["symbol"] = "qmm_vector_kernel<4>"
    json.dump(seq, open(tmp_path / "seq.json", "w"))
    with pytest.raises(SystemExit):
        ps.main(["trace", "--csv", str(tmp_path / "t.csv"), "--seq", str(tmp_path / "seq.json"),
                 "--command", "cmd", "--out", str(tmp_path / "t.md")])


def test_counter_summary_calibrates_and_guards(tmp_path):
    seq = _seq()
    json.dump(seq, open(tmp_path / "seq.json", "w"))
    # the counters read half the bytes (FETCH_SIZE) / all of them (WRITE_SIZE)
    _write_counter(tmp_path / "f.csv", seq, "FETCH_SIZE", 2.0)
    _write_counter(tmp_path / "w.csv", seq, "WRITE_SIZE", 1.0)
    _write_counter(tmp_path / "cf.csv", seq, "FETCH_SIZE", 1.0, copy_kib=(1 << 30) / 1024 / 2)
    _write_counter(tmp_path / "cw.csv", seq, "WRITE_SIZE", 1.0, copy_kib=(1 << 30) / 1024)
    ps.main(["counters", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
             "--copy-fetch", str(tmp_path / "cf.csv"), "--copy-write", str(tmp_path / "cw.csv"),
             "--seq", str(tmp_path / "seq.json"), "--command", "a ;; b", "--out", str(tmp_path / "c.txt")])
    text = open(tmp_path / "c.txt").read()
    assert "FETCH_SIZE x 2.0000, WRITE_SIZE x 1.0000" in text
    assert "passed on every dispatch" in text
    t = dict(re.findall(r"traffic_bytes_per_dispatch\[(.+?)\]: (\d+)", text))
    N, K = SHAPES["lm_head"]
    assert int(t["lm_head M=4"]) == pytest.approx(acc.weight_bytes(N, K) + 4 * 4 * N, abs=1)
    assert "config single_2048 M=4" in t


def test_committed_counters_pass_the_guard():
    # every full-pass and workload dispatch read at least 0.98 x its weight bytes
    path = os.path.join(ROOT, "profiles", "counters_pass_and_configs.txt")
    if not os.path.exists(path):
        pytest.skip("no committed counter summary")
    text = open(path).read()
    assert "passed on every dispatch" in text
    checked = 0
    for key, val in re.findall(r"traffic_bytes_per_dispatch\[(.+?)\]: (\d+)", text):
        m = re.match(r"(?:config )?(\w+) M=(\d+)$", key)
        if not m:
            continue
        N, K = SHAPES[m.group(1)]
        acc.check_counter_bytes(float(val), acc.weight_bytes(N, K), what=key)
        checked += 1
    assert checked >= 20


def _write_pipeline(path, seq, counters):
    # counters: {name: f(launch) -> value per dispatch}; each value split over
    # two dimension rows (summed by the tool), foreign dispatches in between
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        did = 3
        for s in seq["launches"]:
            for name in counters:
                w.writerow([did - 1, "void qmm::zero_u32(unsigned int*, int)", name, 5.0])
            for name, fn in counters.items():
                v = fn(s)
                w.writerow([did, "void qmm::%s(qmm::Args)" % s["symbol"], name, v / 2])
                w.writerow([did, "void qmm::%s(qmm::Args)" % s["symbol"], name, v / 2])
            did += 2


def test_pipeline_summary(tmp_path):
    seq = _seq()
    json.dump(seq, open(tmp_path / "seq.json", "w"))
    tb = lambda s: ps.tile_blocks(s["N"], s["K"])
    # pass A: 110 VALU and 10 MFMA per tile-block, 6 waves resident, 40% waiting, VALU
    # active 2000 against 1000 busy cycles (synthetic values: the tool only divides)
    a = {"SQ_WAVES": lambda s: 1024.0, "SQ_WAVE_CYCLES": lambda s: 6000.0,
         "SQ_BUSY_CU_CYCLES": lambda s: 1000.0, "SQ_WAIT_INST_ANY": lambda s: 2400.0,
         "SQ_ACTIVE_INST_VALU": lambda s: 2000.0,
         "SQ_INSTS_VALU": lambda s: 110.0 * tb(s), "SQ_INSTS_MFMA": lambda s: 10.0 * tb(s),
         "SQ_VALU_MFMA_BUSY_CYCLES": lambda s: 64.0 * tb(s)}
    # pass B: 12 LDS instructions per tile-block, 0.5 conflict cycles each
    b = {"SQ_INSTS_LDS": lambda s: 12.0 * tb(s), "SQ_LDS_BANK_CONFLICT": lambda s: 6.0 * tb(s),
         "SQ_ACTIVE_INST_LDS": lambda s: 300.0, "SQ_BUSY_CU_CYCLES": lambda s: 1000.0}
    _write_pipeline(tmp_path / "a.csv", seq, a)
    _write_pipeline(tmp_path / "b.csv", seq, b)
    ps.main(["pipeline", "--csv", str(tmp_path / "a.csv"), "--seq", str(tmp_path / "seq.json"),
             "--csv", str(tmp_path / "b.csv"), "--seq", str(tmp_path / "seq.json"),
             "--command", "cmd a ;; cmd b", "--out", str(tmp_path / "p.md")])
    text = open(tmp_path / "p.md").read()
    assert "kernel_source_sha256: 0123456789abcdef" in text and "  cmd b" in text
    cells = lambda l: [c.strip() for c in l.strip().strip("|").split("|")]
    rows = {cells(l)[0]: cells(l) for l in text.splitlines() if l.startswith("| ")}
    # columns: key, dispatches, waves, resident, waiting, VALU active, VALU/tb, MFMA/tb,
    # MFMA busy/tb, LDS/tb, conflicts per LDS instruction, LDS active
    r = rows["square M=1"]
    assert r[1] == "2"
    assert r[5] == "-"  # SQ_WAIT_ANY not collected
    assert [float(x) for x in r[3:5] + r[6:13]] == pytest.approx([6.0, 0.4, 2.0, 110, 10, 64, 12, 0.5, 0.3])
    assert rows["qmm_tiled_kernel<1, false, 0>"][1] == "5"
    assert rows["config single_2048 M=4"][1] == "1"
    # a counter missing from every run leaves its column empty
    (tmp_path / "c.csv").write_text(open(tmp_path / "a.csv").read().replace("SQ_INSTS_MFMA", "SQ_OTHER"))
    ps.main(["pipeline", "--csv", str(tmp_path / "c.csv"), "--seq", str(tmp_path / "seq.json"),
             "--command", "c", "--out", str(tmp_path / "q.md")])
    r = [cells(l) for l in open(tmp_path / "q.md").read().splitlines() if l.startswith("| square M=1")][0]
    assert r[8] == "-"


def test_kernel_counters(tmp_path):
    # one kernel's counters over its dispatches; other kernels are ignored
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(tmp_path / "k.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for did in (1, 2):
            for name, v in (("SQ_WAVES", 100.0), ("SQ_WAVE_CYCLES", 5000.0), ("SQ_BUSY_CU_CYCLES", 1000.0),
                            ("SQ_WAIT_ANY", 2000.0 * did), ("SQ_INSTS_VALU", 3000.0)):
                w.writerow([did, "gdn_replay_kernel(float*, ...)", name, v / 2])
                w.writerow([did, "gdn_replay_kernel(float*, ...)", name, v / 2])
            w.writerow([did + 10, "other_kernel", "SQ_WAVES", 7.0])
    ps.main(["kernel-counters", "--csv", str(tmp_path / "k.csv"), "--kernel", "gdn_replay_kernel",
             "--command", "c1 ;; c2", "--out", str(tmp_path / "k.md"), "--sha", "abc"])
    text = open(tmp_path / "k.md").read()
    assert "dispatches: 2" in text and "  c2" in text and "kernel_source_sha256: abc" in text
    assert "SQ_WAVES: 100" in text
    assert "mean waves resident per SIMD: 5" in text
    assert "share of wave time waiting on counters: 0.6" in text  # mean of 2000, 4000 over 5000
    assert "VALU instructions per wave: 30" in text
    assert "VALU active share" not in text  # SQ_ACTIVE_INST_VALU not collected


def _switch_seq(table_kernel):
    # both kernels at 1..4 rows on one shape, two launch shapes each, three launches per shape
    launches = []
    N, K = SHAPES["square"]
    for M in range(1, 5):
        for kernel in ("vector", "tiled"):
            sym = "qmm_vector_kernel<%d>" % M if kernel == "vector" else "qmm_tiled_kernel<1, false, 0>"
            for launch in ("4/2/2", "4/3/1"):
                for _ in range(3):
                    launches.append({"symbol": sym, "shape": "square", "M": M, "N": N, "K": K,
                                     "kernel": kernel, "table_kernel": table_kernel(M),
                                     "launch": launch})
    return {"kernel_source_sha256": "0123456789abcdef", "launches": launches}


def _switch_us(s):
    # row-vector: 6 us + 2 us per row; tiled: 9 us flat; the 4/3/1 shape 1 us slower
    base = 6.0 + 2.0 * s["M"] if s["kernel"] == "vector" else 9.0
    return base + (1.0 if s["launch"] == "4/3/1" else 0.0)


def _write_switch_trace(path, seq):
    cols = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        t = 1000
        for did, s in enumerate(seq["launches"], start=1):
            w.writerow(["KERNEL_DISPATCH", did, "void qmm::%s(qmm::Args)" % s["symbol"], t,
                        t + int(_switch_us(s) * 1000)])
            t += 10 ** 6


@pytest.mark.parametrize("table_from", [2, 1])
def test_switch_summary(tmp_path, table_from):
    # the tiled kernel is faster from 2 rows (8 + 2 = 10 > 9 us); a table that
    # switches at 1 row disagrees with the measurement at M = 1
    seq = _switch_seq(lambda M: "tiled" if M >= table_from else "vector")
    json.dump(seq, open(tmp_path / "seq.json", "w"))
    _write_switch_trace(tmp_path / "trace.csv", seq)
    out = tmp_path / "switch.md"
    ps.main(["switch", "--csv", str(tmp_path / "trace.csv"), "--seq", str(tmp_path / "seq.json"),
             "--command", "rocprofv3 ... -- python3 bench.py --mode switch", "--out", str(out)])
    text = out.read_text()
    rows = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 8 and cells[0] == "square":
            rows[int(cells[1])] = cells
    assert sorted(rows) == [1, 2, 3, 4]
    assert rows[1][2] == "8.000 (4/2/2)" and rows[1][3] == "9.000 (4/2/2)"
    assert rows[1][5] == "vector" and all(rows[m][5] == "tiled" for m in (2, 3, 4))
    assert rows[4][4] == "%.3f" % (9.0 / 14.0)
    assert float(rows[2][7]) == pytest.approx(acc.weight_bytes(5120, 5120) / 9e-6 / 1e9, rel=1e-3)
    assert "switch_point[square]: 2" in text
    assert ("table_agrees_with_measurement: yes" in text) == (table_from == 2)

"""Summaries of rocprofv3 runs of `bench.py --mode kernels`, per kernel and per
(matrix shape, row count).

bench.py --mode kernels --seq-out SEQ launches one event-timed eager pass per
row count and two calls of each single-matrix workload per row count, and
writes the sequence of its launches (kernel symbol, shape, M) to SEQ. The
profiler's dispatches of the library's kernels come in the same order, so
each one can be named by its shape and row count:

  trace:    python -m skinny_bit_block_amd.profile_summary trace --csv <kernel_trace.csv>
                [--stats <kernel_stats.csv>] --seq SEQ --command "..."
                --out profiles/kernels_trace_pass_and_configs.md
  counters: python -m skinny_bit_block_amd.profile_summary counters --fetch <csv> --write <csv>
                --copy-fetch <csv> --copy-write <csv> --seq SEQ --command "..."
                --out profiles/counters_pass_and_configs.txt
  pipeline: python -m skinny_bit_block_amd.profile_summary pipeline --csv <csv> --seq SEQ
                [--csv <csv> --seq SEQ ...] --command "..."
                --out profiles/pipeline_counters_pass_and_configs.md
  switch:   python -m skinny_bit_block_amd.profile_summary switch --csv <kernel_trace.csv>
                --seq SEQ --command "..." --out profiles/switch_point_vector_vs_tiled.md
                (SEQ from bench.py --mode switch: both kernels forced at 1..8 rows)
  kernel-counters: python -m skinny_bit_block_amd.profile_summary kernel-counters
                --csv <csv> [--csv <csv> ...] --kernel NAME --command "..." --out FILE
                (one kernel's counters averaged over its dispatches, any workload)

Counter bytes are calibrated against a plain device copy of known size (bench.py
--mode copy, 1 GiB): FETCH_SIZE and WRITE_SIZE are scaled so that the copy
reads and writes exactly its size. The counter summary ends with
"traffic_bytes_per_dispatch[key]: bytes" lines (key = kernel symbol, "shape
M=m" or "config shape M=m"), which bench.py reads back when the kernel source
has not changed since, and it applies the accounting's counter guard (counter
bytes below 0.98 x the weight bytes mean a cache served the weights).
"""
import argparse
import csv
import json
import re
import sys

from . import accounting as acc

_SYM = re.compile(r"(qmm_(?:vector|tiled)_kernel<[^>]*>)")


def _col(row, *names):
    low = {k.lower(): k for k in row}
    for n in names:
        if n.lower() in low:
            return row[low[n.lower()]]
    raise KeyError(names)


def _symbol(name):
    m = _SYM.search(name)
    return m.group(1) if m else None


def _dispatches(path):
    """[(dispatch id, symbol, row)] of the library's kernels, in dispatch order."""
    out = []
    with open(path) as f:
        for row in csv.DictReader(f):
            sym = _symbol(_col(row, "Kernel_Name", "KernelName"))
            if sym:
                out.append((int(_col(row, "Dispatch_Id", "Dispatch_ID", "DispatchId")), sym, row))
    out.sort(key=lambda t: t[0])
    return out


def _align(disp, seq):
    """Name each dispatch by its launch; the symbols must agree one by one."""
    if len(disp) != len(seq):
        raise SystemExit("%d library dispatches but %d launches in the sequence" % (len(disp), len(seq)))
    for (did, sym, _), s in zip(disp, seq):
        if sym != s["symbol"]:
            raise SystemExit("dispatch %d is %s, the sequence has %s" % (did, sym, s["symbol"]))
    return list(zip(disp, seq))


def _key(s):
    return "%s M=%d" % (s["shape"], s["M"])


def _config(s):
    # launches of the single-matrix workloads; the rest are the full passes
    return s["shape"].startswith("config ")


def trace(args):
    seq = json.load(open(args.seq))
    pairs = _align(_dispatches(args.csv), seq["launches"])
    by_sym, by_key = {}, {}
    for (did, sym, row), s in pairs:
        us = (int(_col(row, "End_Timestamp", "EndNs")) - int(_col(row, "Start_Timestamp", "BeginNs"))) * 1e-3
        keys = ((_key(s), by_key),) if _config(s) else ((sym, by_sym), (_key(s), by_key))
        for k, t in keys:
            d = t.setdefault(k, {"n": 0, "us": 0.0, "wb": 0, "ab": 0, "min": 1e30, "max": 0.0})
            d["n"] += 1
            d["us"] += us
            d["min"] = min(d["min"], us)
            d["max"] = max(d["max"], us)
            d["wb"] += acc.weight_bytes(s["N"], s["K"])
            d["ab"] += acc.call_bytes(s["M"], s["N"], s["K"])
    lines = ["# rocprofv3 kernel trace: event-timed eager launches of bench.py --mode kernels", "",
             "command (repository root, after cd /tmp && export TMPDIR=/tmp):", "  " + args.command,
             "kernel_source_sha256: %s" % seq["kernel_source_sha256"], "",
             "Per kernel, over the launches of the full passes (one eager pass at each M): algorithmic",
             "bytes per launch (weights + fp32 x + fp32 y) over the mean kernel duration. The bench",
             "line's roofline divides the same bytes by its own event-timed mean of the same launches.", "",
             "| kernel | dispatches | mean us | min us | max us | algorithmic GB/s | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|"]
    for k, d in sorted(by_sym.items()):
        mean = d["us"] / d["n"]
        gbs = d["ab"] / d["n"] / (mean * 1e-6) / 1e9
        lines.append("| %s | %d | %.3f | %.3f | %.3f | %.1f | %.2f |"
                     % (k, d["n"], mean, d["min"], d["max"], gbs, gbs / 80.0))
    lines += ["", "Per shape and row count (weight bytes only; \"config\" rows are the single-matrix",
              "workloads, two calls on distinct copies per M):", "",
              "| shape, M | dispatches | mean us | weight GB/s | % of 8 TB/s |", "|---|---|---|---|---|"]
    for k, d in sorted(by_key.items()):
        mean = d["us"] / d["n"]
        gbs = d["wb"] / d["n"] / (mean * 1e-6) / 1e9
        lines.append("| %s | %d | %.3f | %.1f | %.2f |" % (k, d["n"], mean, gbs, gbs / 80.0))
    if args.stats:
        lines += ["", "rocprofv3 --stats of the same run (every dispatch of the program: the full passes",
                  "and the single-matrix workloads together):", "",
                  "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
        with open(args.stats) as f:
            for row in csv.DictReader(f):
                name = _symbol(row["Name"]) or row["Name"][:60]
                lines.append("| %s | %s | %.3f | %.3f | %.3f | %.2f |" % (
                    name, row["Calls"], float(row["AverageNs"]) * 1e-3, float(row["MinNs"]) * 1e-3,
                    float(row["MaxNs"]) * 1e-3, float(row["Percentage"])))
        lines.append("")
    for k, d in sorted(by_sym.items()):
        lines.append("mean_kernel_us[%s]: %.3f" % (k, d["us"] / d["n"]))
    open(args.out, "w").write("\n".join(lines) + "\n")


def _counter(path, name):
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if _col(row, "Counter_Name", "CounterName") != name:
                continue
            did = int(_col(row, "Dispatch_Id", "Dispatch_ID", "DispatchId"))
            vals[did] = vals.get(did, 0.0) + float(_col(row, "Counter_Value", "CounterValue"))
    return vals


def _copy_kib(path, name):
    vals = []
    with open(path) as f:
        for row in csv.DictReader(f):
            if "copyBuffer" in _col(row, "Kernel_Name", "KernelName") and \
                    _col(row, "Counter_Name", "CounterName") == name:
                vals.append(float(_col(row, "Counter_Value", "CounterValue")))
    if not vals:
        raise SystemExit("no copy dispatch with %s in %s" % (name, path))
    return sum(vals) / len(vals)


def counters(args):
    seq = json.load(open(args.seq))
    fetch = _counter(args.fetch, "FETCH_SIZE")
    write = _counter(args.write, "WRITE_SIZE")
    copy_bytes = 1 << 30
    ff = copy_bytes / 1024.0 / _copy_kib(args.copy_fetch, "FETCH_SIZE")
    wf = copy_bytes / 1024.0 / _copy_kib(args.copy_write, "WRITE_SIZE")
    # the counter CSV has one row per (dispatch, counter): keep one entry per dispatch
    seen, disp = set(), []
    for did, sym, row in _dispatches(args.fetch):
        if did not in seen:
            seen.add(did)
            disp.append((did, sym, row))
    pairs = _align(disp, seq["launches"])
    # the WRITE_SIZE run dispatches the same sequence: pair its library dispatches by position
    wdisp = sorted({int(_col(r, "Dispatch_Id", "Dispatch_ID", "DispatchId")) for _, _, r in _dispatches(args.write)})
    if len(wdisp) != len(disp):
        raise SystemExit("%d library dispatches in the FETCH_SIZE run, %d in the WRITE_SIZE run"
                         % (len(disp), len(wdisp)))
    by = {}
    guard = []
    for i, ((did, sym, row), s) in enumerate(pairs):
        fb = fetch[did] * 1024.0 * ff
        wb_ = write[wdisp[i]] * 1024.0 * wf
        for k in ((_key(s),) if _config(s) else (sym, _key(s))):
            d = by.setdefault(k, {"n": 0, "f": 0.0, "w": 0.0, "wb": 0, "ab": 0})
            d["n"] += 1
            d["f"] += fb
            d["w"] += wb_
            d["wb"] += acc.weight_bytes(s["N"], s["K"])
            d["ab"] += acc.call_bytes(s["M"], s["N"], s["K"])
        try:
            acc.check_counter_bytes(fb, acc.weight_bytes(s["N"], s["K"]), what=_key(s))
        except acc.RooflineViolation as e:
            guard.append(str(e))
    lines = ["# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
             "workload: bench.py --mode kernels (one eager pass at each M, two calls of each "
             "single-matrix workload per M)",
             "kernel_source_sha256: %s" % seq["kernel_source_sha256"],
             "commands (repository root, after cd /tmp && export TMPDIR=/tmp):"]
    lines += ["  " + c for c in args.command.split(" ;; ")]
    lines += ["calibration (plain 1 GiB device copy): FETCH_SIZE x %.4f, WRITE_SIZE x %.4f" % (ff, wf),
              "counter guard (counter bytes >= 0.98 x weight bytes per dispatch): %s"
              % ("passed on every dispatch" if not guard else "FAILED: " + "; ".join(guard[:5])),
              "",
              "(kernel keys: the full-pass launches; \"config\" keys: the single-matrix workloads)",
              "key | dispatches | fetch bytes | write bytes | traffic/dispatch | algorithmic/dispatch | ratio"]
    for k, d in sorted(by.items()):
        t = (d["f"] + d["w"]) / d["n"]
        a = d["ab"] / d["n"]
        lines.append("%s | %d | %.0f | %.0f | %.0f | %.0f | %.3f" % (k, d["n"], d["f"] / d["n"],
                                                                      d["w"] / d["n"], t, a, t / a))
    for k, d in sorted(by.items()):
        lines.append("traffic_bytes_per_dispatch[%s]: %.0f" % (k, (d["f"] + d["w"]) / d["n"]))
    open(args.out, "w").write("\n".join(lines) + "\n")
    if guard:
        sys.stderr.write("counter guard failed on %d dispatches\n" % len(guard))


def stats(args):
    """One kernel's rocprofv3 figures: the --stats row of a kernel-trace run,
    and, when counter runs are given, its calibrated FETCH_SIZE / WRITE_SIZE
    bytes per dispatch against its algorithmic bytes."""
    want = args.kernel
    lines = ["# rocprofv3 summary: %s" % want, "", "commands (repository root, after cd /tmp && "
             "export TMPDIR=/tmp):"]
    lines += ["  " + c for c in args.command.split(" ;; ")]
    if args.sha:
        lines.append("kernel_source_sha256: %s" % args.sha)
    lines.append("")
    with open(args.stats) as f:
        for row in csv.DictReader(f):
            if want in row["Name"]:
                lines += ["| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|",
                          "| %s | %s | %.3f | %.3f | %.3f |" % (want, row["Calls"], float(row["AverageNs"]) * 1e-3,
                                                            float(row["MinNs"]) * 1e-3, float(row["MaxNs"]) * 1e-3)]
                avg_us = float(row["AverageNs"]) * 1e-3
                break
        else:
            raise SystemExit("%s not in %s" % (want, args.stats))
    lines.append("mean_kernel_us[%s]: %.3f" % (want, avg_us))
    if args.fetch:
        def per_dispatch(path, name):
            vals = {}
            with open(path) as f:
                for row in csv.DictReader(f):
                    if want in _col(row, "Kernel_Name", "KernelName") and _col(row, "Counter_Name", "CounterName") == name:
                        did = int(_col(row, "Dispatch_Id", "Dispatch_ID", "DispatchId"))
                        vals[did] = vals.get(did, 0.0) + float(_col(row, "Counter_Value", "CounterValue"))
            return list(vals.values())
        ff = (1 << 30) / 1024.0 / _copy_kib(args.copy_fetch, "FETCH_SIZE")
        wf = (1 << 30) / 1024.0 / _copy_kib(args.copy_write, "WRITE_SIZE")
        fv, wv = per_dispatch(args.fetch, "FETCH_SIZE"), per_dispatch(args.write, "WRITE_SIZE")
        fb = sum(fv) / len(fv) * 1024.0 * ff
        wb = sum(wv) / len(wv) * 1024.0 * wf
        lines += ["", "calibration (plain 1 GiB device copy): FETCH_SIZE x %.4f, WRITE_SIZE x %.4f" % (ff, wf),
                  "dispatches: %d (fetch run), %d (write run)" % (len(fv), len(wv)),
                  "fetch bytes per dispatch: %.0f" % fb, "write bytes per dispatch: %.0f" % wb]
        if args.algorithmic:
            lines.append("algorithmic bytes per dispatch: %d (ratio %.3f)"
                         % (args.algorithmic, (fb + wb) / args.algorithmic))
        lines.append("traffic_bytes_per_dispatch[%s]: %.0f" % (want, fb + wb))
    open(args.out, "w").write("\n".join(lines) + "\n")


# Pipeline counters of the library's kernels (rocprofv3 --pmc, raw SQ counters
# in passes within the hardware's per-pass limits). A tile-block is one
# 16-row tile times one 256-weight super-block: a wave's unit of work, so the
# per-tile-block figures compare launch shapes and row counts directly.
PIPELINE = [
    # (label, how it is formed from the counters of one dispatch)
    ("waves", lambda c, tb: c["SQ_WAVES"]),
    ("mean waves resident per SIMD", lambda c, tb: c["SQ_WAVE_CYCLES"] / c["SQ_BUSY_CU_CYCLES"]),
    ("share of wave time waiting to issue", lambda c, tb: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
    ("share of wave time waiting on counters", lambda c, tb: c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]),
    ("VALU active share of busy SIMD time",
     lambda c, tb: c["SQ_ACTIVE_INST_VALU"] / c["SQ_BUSY_CU_CYCLES"]),
    ("VALU instructions per tile-block", lambda c, tb: c["SQ_INSTS_VALU"] / tb),
    ("MFMA instructions per tile-block", lambda c, tb: c["SQ_INSTS_MFMA"] / tb),
    ("MFMA busy cycles per tile-block", lambda c, tb: c["SQ_VALU_MFMA_BUSY_CYCLES"] / tb),
    ("LDS instructions per tile-block", lambda c, tb: c["SQ_INSTS_LDS"] / tb),
    ("LDS bank-conflict cycles per LDS instruction",
     lambda c, tb: c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_INSTS_LDS"], 1.0)),
    ("LDS active share of busy CU time",
     lambda c, tb: c["SQ_ACTIVE_INST_LDS"] / c["SQ_BUSY_CU_CYCLES"]),
]


def _all_counters(path):
    """{dispatch id: {counter: value summed over its dimensions}} of the library's kernels."""
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if not _symbol(_col(row, "Kernel_Name", "KernelName")):
                continue
            did = int(_col(row, "Dispatch_Id", "Dispatch_ID", "DispatchId"))
            name = _col(row, "Counter_Name", "CounterName")
            d = vals.setdefault(did, {})
            d[name] = d.get(name, 0.0) + float(_col(row, "Counter_Value", "CounterValue"))
    return vals


def tile_blocks(N, K):
    return (N + 15) // 16 * (K // acc.BLOCK_WEIGHTS)


def pipeline(args):
    if len(args.csv) != len(args.seq):
        raise SystemExit("one --seq per --csv")
    by = {}
    sha = None
    for path, seqp in zip(args.csv, args.seq):
        seq = json.load(open(seqp))
        sha = seq["kernel_source_sha256"]
        vals = _all_counters(path)
        seen, disp = set(), []
        for did, sym, row in _dispatches(path):
            if did not in seen:
                seen.add(did)
                disp.append((did, sym, row))
        for (did, sym, _), s in _align(disp, seq["launches"]):
            for k in ((_key(s),) if _config(s) else (sym, _key(s))):
                d = by.setdefault(k, {"n": {}, "c": {}, "tb": 0.0, "ntb": 0})
                for name, v in vals[did].items():
                    d["c"][name] = d["c"].get(name, 0.0) + v
                    d["n"][name] = d["n"].get(name, 0) + 1
                if path == args.csv[0]:
                    d["tb"] += tile_blocks(s["N"], s["K"])
                    d["ntb"] += 1
    lines = ["# Pipeline counters per dispatch (rocprofv3 --pmc, raw SQ counters)", "",
             "workload: bench.py --mode kernels (one eager pass at each M, two calls of each "
             "single-matrix workload per M)",
             "kernel_source_sha256: %s" % sha,
             "commands (repository root, after cd /tmp && export TMPDIR=/tmp):"]
    lines += ["  " + c for c in args.command.split(" ;; ")]
    lines += ["", "Per dispatch means; a tile-block is one 16-row tile x one 256-weight super-block",
              "(ceil(N/16) K/256 per matrix). Ratios: resident waves = SQ_WAVE_CYCLES /",
              "SQ_BUSY_CU_CYCLES, which reads 1.0 for launch shapes with one 4-wave workgroup per",
              "busy CU, i.e. waves per SIMD; waiting to issue = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES;",
              "waiting on counters (s_waitcnt: memory, LDS) = SQ_WAIT_ANY / SQ_WAVE_CYCLES; VALU active",
              "= SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES; LDS active = SQ_ACTIVE_INST_LDS /",
              "SQ_BUSY_CU_CYCLES; bank-conflict cycles per LDS instruction = SQ_LDS_BANK_CONFLICT /",
              "SQ_INSTS_LDS. (kernel keys: the full-pass launches; \"config\" keys: the single-matrix",
              "workloads)", ""]
    labels = [l for l, _ in PIPELINE]
    lines.append("| key | dispatches | " + " | ".join(labels) + " |")
    lines.append("|---|---|" + "---|" * len(labels))
    for k, d in sorted(by.items()):
        c = {name: v / d["n"][name] for name, v in d["c"].items()}
        tb = d["tb"] / max(d["ntb"], 1)
        cells = []
        for _, f in PIPELINE:
            try:
                v = f(c, tb)
                cells.append("%.0f" % v if abs(v) >= 100 else "%.3g" % v)
            except (KeyError, ZeroDivisionError):
                cells.append("-")
        lines.append("| %s | %d | %s |" % (k, d["ntb"], " | ".join(cells)))
    open(args.out, "w").write("\n".join(lines) + "\n")


def kernel_counters(args):
    """Pipeline counters of one kernel (any symbol containing --kernel), averaged
    over its dispatches in one or more counter runs, with the same ratios as
    the pipeline summary (per wave instead of per tile-block)."""
    per = {}
    for path in args.csv:
        with open(path) as f:
            for row in csv.DictReader(f):
                if args.kernel not in _col(row, "Kernel_Name", "KernelName"):
                    continue
                key = (path, int(_col(row, "Dispatch_Id", "Dispatch_ID", "DispatchId")))
                d = per.setdefault(key, {})
                name = _col(row, "Counter_Name", "CounterName")
                d[name] = d.get(name, 0.0) + float(_col(row, "Counter_Value", "CounterValue"))
    if not per:
        raise SystemExit("no dispatch of %s" % args.kernel)
    tot, cnt = {}, {}
    for d in per.values():
        for k, v in d.items():
            tot[k] = tot.get(k, 0.0) + v
            cnt[k] = cnt.get(k, 0) + 1
    c = {k: tot[k] / cnt[k] for k in tot}
    lines = ["# Pipeline counters: %s" % args.kernel, "",
             "commands (repository root, after cd /tmp && export TMPDIR=/tmp):"]
    lines += ["  " + x for x in args.command.split(" ;; ")]
    if args.sha:
        lines.append("kernel_source_sha256: %s" % args.sha)
    lines += ["", "dispatches: %d (means per dispatch; counters summed over their dimensions)"
              % (len(per) // max(len(args.csv), 1)), ""]
    for k in sorted(c):
        lines.append("%s: %.6g" % (k, c[k]))
    ratios = [
        ("mean waves resident per SIMD", "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES"),
        ("share of wave time waiting on counters", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
        ("share of wave time waiting to issue", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
        ("VALU active share of busy SIMD time", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CU_CYCLES"),
        ("LDS active share of busy CU time", "SQ_ACTIVE_INST_LDS", "SQ_BUSY_CU_CYCLES"),
        ("VALU instructions per wave", "SQ_INSTS_VALU", "SQ_WAVES"),
    ]
    lines.append("")
    for label, a, b in ratios:
        if a in c and b in c and c[b]:
            lines.append("%s: %.4g" % (label, c[a] / c[b]))
    open(args.out, "w").write("\n".join(lines) + "\n")


def switch(args):
    """The row-vector (VALU dot2) / tiled (MFMA) comparison of bench.py --mode
    switch: per (shape, M, kernel) the mean kernel duration of each launch shape
    tried, the faster kernel with its best shape, and the row count from which
    the tiled kernel stays faster, against the launch table's choice."""
    seq = json.load(open(args.seq))
    pairs = _align(_dispatches(args.csv), seq["launches"])
    runs, table, dims = {}, {}, {}
    for (did, sym, row), s in pairs:
        us = (int(_col(row, "End_Timestamp", "EndNs")) - int(_col(row, "Start_Timestamp", "BeginNs"))) * 1e-3
        d = runs.setdefault((s["shape"], s["M"], s["kernel"], s["launch"]), [])
        d.append(us)
        table[(s["shape"], s["M"])] = s["table_kernel"]
        dims[s["shape"]] = (s["N"], s["K"])
    best = {}
    for (shape, M, kernel, launch), v in runs.items():
        mean = sum(v) / len(v)
        cur = best.get((shape, M, kernel))
        if cur is None or mean < cur[0]:
            best[(shape, M, kernel)] = (mean, launch, len(v))
    lines = ["# Switch point: row-vector kernel (VALU dot2) against tiled kernel (MFMA)", "",
             "command (repository root, after cd /tmp && export TMPDIR=/tmp):", "  " + args.command,
             "kernel_source_sha256: %s" % seq["kernel_source_sha256"], "",
             "rocprofv3 kernel-trace durations of bench.py --mode switch: each kernel forced at 1..8",
             "rows on every matrix shape of the pass, with every launch shape (waves/K slices/slices",
             "per workgroup) of the table's entries for the matrix that fits at M rows, each launched",
             "three times on distinct cold copies of the matrix. Per kernel the fastest shape's mean;",
             "weight GB/s = weight bytes / that mean.", "",
             "| shape | M | row-vector us (shape) | tiled us (shape) | tiled / row-vector | "
             "faster | table's kernel | weight GB/s of the faster |",
             "|---|---|---|---|---|---|---|---|"]
    shapes = sorted({k[0] for k in best}, key=lambda sh: list(dims).index(sh))
    agree = True
    summary = []
    for shape in shapes:
        N, K = dims[shape]
        first = None
        for M in sorted({k[1] for k in best if k[0] == shape}):
            v, t = best.get((shape, M, "vector")), best.get((shape, M, "tiled"))
            if v is None or t is None:
                continue
            faster = "tiled" if t[0] < v[0] else "vector"
            if faster == "tiled" and first is None:
                first = M
            elif faster == "vector":
                first = None
            if faster != table[(shape, M)]:
                agree = False
            gbs = acc.weight_bytes(N, K) / (min(v[0], t[0]) * 1e-6) / 1e9
            lines.append("| %s | %d | %.3f (%s) | %.3f (%s) | %.3f | %s | %s | %.1f |" % (
                shape, M, v[0], v[1], t[0], t[1], t[0] / v[0], faster, table[(shape, M)], gbs))
        summary.append((shape, first))
    lines += ["", "Row count from which the tiled kernel is faster at every measured M (none: the",
              "row-vector kernel wins somewhere at the top):", ""]
    for shape, first in summary:
        lines.append("switch_point[%s]: %s" % (shape, first if first is not None else "none"))
    lines.append("table_agrees_with_measurement: %s" % ("yes" if agree else "no"))
    open(args.out, "w").write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--csv", required=True)
    t.add_argument("--seq", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--stats", default="", help="rocprofv3's kernel_stats.csv of the same run")
    c = sub.add_parser("counters")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--seq", "--command", "--out"):
        c.add_argument(a, required=True)
    st = sub.add_parser("stats")
    st.add_argument("--kernel", required=True)
    st.add_argument("--stats", required=True)
    st.add_argument("--command", required=True)
    st.add_argument("--out", required=True)
    st.add_argument("--sha", default="")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        st.add_argument(a, default="")
    st.add_argument("--algorithmic", type=int, default=0)
    pp = sub.add_parser("pipeline")
    pp.add_argument("--csv", action="append", required=True, help="a counter_collection.csv (repeat)")
    pp.add_argument("--seq", action="append", required=True, help="its launch sequence (repeat)")
    pp.add_argument("--command", required=True)
    pp.add_argument("--out", required=True)
    kc = sub.add_parser("kernel-counters")
    kc.add_argument("--csv", action="append", required=True, help="a counter_collection.csv (repeat)")
    kc.add_argument("--kernel", required=True)
    kc.add_argument("--command", required=True)
    kc.add_argument("--out", required=True)
    kc.add_argument("--sha", default="")
    sw = sub.add_parser("switch")
    sw.add_argument("--csv", required=True)
    sw.add_argument("--seq", required=True)
    sw.add_argument("--command", required=True)
    sw.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    {"trace": trace, "counters": counters, "stats": stats, "pipeline": pipeline,
     "kernel-counters": kernel_counters, "switch": switch}[args.what](args)


if __name__ == "__main__":
    main()

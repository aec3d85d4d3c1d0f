#!/usr/bin/env python3
"""Benchmark of the skinny quantized product on one MI355X.

Default mode (the contract): one step = one full model pass at each of
M = 1, 4, 8, 16 rows. A pass is 513 calls back-to-back on one stream: per layer
(64) six 5120x5120 projections, the fused gate+up (34816x5120) and the down
projection (5120x17408), then the 151936x5120 lm_head: 15,725,813,760 bytes of
4.5-bit super-blocks, every matrix distinct and resident in HBM before timing.
Prints one JSON line: weight GB/s over the step (value), ms per pass per M, and
in the same run: the 32-row pass, a fused-projection pass (each layer's five
same-input projections as one 25600-row call: 257 calls over the same bytes),
the four single-matrix workloads per row count, the memory-system probes
(stream-read ceiling, sustained read, launch gap, shader clock), per-(shape, M) kernel
durations, the roofline of the dominant kernel and the oracle timed on the
host cores on a bounded sample.

Kernel durations are the kernels' own execution times: every timed launch
records HIP events at the start and end of the kernel itself (the library's
qmm_set_launch_events hook), which is what rocprofv3's kernel trace measures.

Other modes: --mode configs (the single-matrix workloads only), --mode kernels
(only the event-timed eager launches, for rocprofv3 runs; --seq-out writes
the launch sequence that skinny_bit_block_amd/profile_summary.py maps the
trace onto), --mode switch (both kernels forced at 1..8 rows on every pass
shape, for the rocprofv3 run behind the switch point), --mode copy (a plain
device copy of known size, the calibration of the FETCH_SIZE / WRITE_SIZE
counters).
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weight GB/s (% HBM peak) and ms per 15.8 GB pass at M=1,4,8,16"
PEAK_GBS = 8000.0
SEED = 20261202
KERNEL_SRCS = [os.path.join(ROOT, "skinny_bit_block_amd", "csrc", f)
               for f in ("qmm_kernels.hip", "qmm_internal.h", "qmm_api.cpp")]


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def kernel_source_sha():
    """Hash of the kernels and the launch table: a profile taken on other source
    does not describe these launches."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--ms", default="1,4,8,16")
    ap.add_argument("--extra-ms", default="32",
                    help="row counts also timed per pass but not part of value ('' for none)")
    ap.add_argument("--mode", default="pass", choices=["pass", "configs", "kernels", "switch", "copy", "gdn"])
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ids", action="store_true", help="skip the expert-indexed record")
    ap.add_argument("--no-fp4", action="store_true", help="skip the block-scaled FP4 record")
    ap.add_argument("--no-int4", action="store_true", help="skip the plain INT4 record")
    ap.add_argument("--no-eager", action="store_true")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-projection pass")
    ap.add_argument("--no-configs", action="store_true", help="skip the single-matrix workloads")
    ap.add_argument("--no-probes", action="store_true", help="skip the memory-system probes")
    ap.add_argument("--no-gdn", action="store_true", help="skip the recurrent-update record")
    ap.add_argument("--seq-out", default="", help="--mode kernels / switch: write the launch sequence here")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--layers", type=int, default=64, help="(for quick tests only; the metric needs 64)")
    return ap.parse_args()


# the single-matrix workloads: (name, N, K, row counts, activation scale)
CONFIGS = [("single 2048x2048", 2048, 2048, [4], 1.0),
           ("gate+up 34816x5120", 34816, 5120, [1, 2, 4, 7, 8, 9, 16], 1.0),
           ("down 5120x17408", 5120, 17408, [1, 4, 8, 16], 0.1),
           ("lm_head 151936x5120", 151936, 5120, [1, 7], 1.0)]


def shape_class(N, K):
    return {(5120, 5120): "square", (34816, 5120): "gate_up", (5120, 17408): "down",
            (151936, 5120): "lm_head", (25600, 5120): "fused_5x5120", (2048, 2048): "single_2048"}.get(
        (N, K), "%dx%d" % (N, K))


class Pass:
    """Device-resident weights, activations and outputs of one full model pass.

    The arena holds each layer's six 5120x5120 projections back to back, then
    its gate+up and down projection (each at a 2 MiB-aligned start), then the
    lm_head, the way an inference engine keeps its weights. The first five
    projections of a layer therefore also form one contiguous 25600x5120
    matrix: the fused-projection pass calls that once (they share one input in
    the layer) and the sixth separately, over exactly the same bytes.
    """

    def __init__(self, torch, sbb, synth, acc, ms, layers):
        import numpy as np
        self.torch, self.sbb = torch, sbb
        self.shapes = [s for s in acc.full_pass_shapes()
                       if s[0] == "lm_head" or int(s[0][1:].split(".")[0]) < layers]
        self.weight_bytes = sum(acc.weight_bytes(N, K) for _, N, K in self.shapes)
        self.ms = ms
        dev = torch.device("cuda:0")
        align = 2 << 20
        offs, total = [], 0
        for i, (name, N, K) in enumerate(self.shapes):
            contiguous = ".proj" in name and not name.endswith(".proj0")
            if not contiguous:
                total = -(-total // align) * align
            offs.append(total)
            total += acc.weight_bytes(N, K)
        self.arena = torch.empty(-(-total // align) * align, dtype=torch.uint8, device=dev)
        self.W = []
        bufs = {}
        t0 = time.time()
        for i, (name, N, K) in enumerate(self.shapes):
            nbytes = acc.weight_bytes(N, K)
            if nbytes not in bufs:
                bufs[nbytes] = np.empty(nbytes, dtype=np.uint8)
            host = bufs[nbytes]
            synth.weights(N, K, tensor=i + 1, seed=SEED, out=host.reshape(N, -1))
            d = self.arena[offs[i]:offs[i] + nbytes]
            d.copy_(torch.from_numpy(host))
            self.W.append(d)
            if i % 64 == 0:
                log("weights %d/%d resident (%.1f s)" % (i + 1, len(self.shapes), time.time() - t0))
        torch.cuda.synchronize()
        log("all %d matrices resident: %.3f GB in %.1f s"
            % (len(self.shapes), self.weight_bytes / 1e9, time.time() - t0))
        self.x = {}
        self.y = {}
        Ns = sorted({N for _, N, _ in self.shapes} | {5 * 5120})
        for M in ms:
            for K in sorted({K for _, _, K in self.shapes}):
                xs = synth.acts(M, K, tensor=100000 + K, seed=SEED)
                self.x[(M, K)] = torch.from_numpy(xs).to(dev)
            for N in Ns:
                self.y[(M, N)] = torch.empty((M, N), dtype=torch.float32, device=dev)
        self.lib = sbb.load()
        self.h = sbb.qmm_create(0)
        self.calls = {}
        self.fused_calls = {}
        vp = ctypes.c_void_p
        for M in ms:
            lst, fl = [], []
            for (name, N, K), Wd in zip(self.shapes, self.W):
                c = (vp(self.x[(M, K)].data_ptr()), vp(Wd.data_ptr()), vp(self.y[(M, N)].data_ptr()), M, N, K)
                lst.append(c)
                if name.endswith(".proj0"):  # projections 0..4 as one 25600-row call
                    fl.append((c[0], c[1], vp(self.y[(M, 5 * 5120)].data_ptr()), M, 5 * N, K))
                elif ".proj" in name and not name.endswith(".proj5"):
                    continue
                else:
                    fl.append(c)
            self.calls[M] = lst
            self.fused_calls[M] = fl
        self.graphs = {}
        self.fused_graphs = {}

    def run(self, M, stream_ptr, fused=False):
        fn, h = self.lib.qmm_run, self.h
        s = ctypes.c_void_p(stream_ptr)
        for x, w, y, m, n, k in (self.fused_calls if fused else self.calls)[M]:
            rc = fn(h, x, w, y, m, n, k, s)
            if rc:
                raise RuntimeError("qmm_run failed: %s" % self.sbb.qmm_status_string(rc))

    def capture(self, fused=False, ms=None):
        torch = self.torch
        graphs = self.fused_graphs if fused else self.graphs
        for M in (self.ms if ms is None else ms):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.run(M, side.cuda_stream, fused)  # warm the kernels outside the capture
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                self.run(M, torch.cuda.current_stream().cuda_stream, fused)
            graphs[M] = g
        torch.cuda.synchronize()

    def plan(self, M, N, K):
        return self.sbb.qmm_query_plan(self.h, M, N, K)

    def kernel_symbol(self, M, N, K):
        p = self.plan(M, N, K)
        if p["kernel"] == self.sbb.KERNEL_TILED:
            return "qmm_tiled_kernel<%d, false, 0>" % (1 if M <= 16 else 2)
        return "qmm_vector_kernel<%d>" % M


def time_passes(P, steps, warmup, graph, ms=None, fused=False):
    """Per-M ms per pass (for the row counts ms, default all of P's), timed with
    HIP events on the stream the kernels run on."""
    torch = P.torch
    stream = torch.cuda.current_stream()
    ms = P.ms if ms is None else ms
    graphs = P.fused_graphs if fused else P.graphs
    ev = {M: [] for M in ms}

    def one_step(record):
        for M in ms:
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            if graph:
                graphs[M].replay()
            else:
                P.run(M, stream.cuda_stream, fused)
            if record:
                b.record(stream)
                ev[M].append((a, b))

    for _ in range(warmup):
        one_step(False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    w0 = time.time()
    t0.record(stream)
    for _ in range(steps):
        one_step(True)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.time() - w0
    total_ms = t0.elapsed_time(t1)
    per_m = {M: sum(a.elapsed_time(b) for a, b in ev[M]) / steps for M in ms}
    return total_ms / steps, per_m, wall


def kernel_timing(P, M_list, seq=None):
    """One eager pass per M in which every launch records HIP events at the
    start and end of its own kernel (qmm_set_launch_events): per-symbol and
    per-(shape, M) launch counts, mean kernel durations and algorithmic bytes.
    seq, if a list, receives the launch sequence (symbol, shape, M) in order."""
    from skinny_bit_block_amd import accounting as acc
    from skinny_bit_block_amd.events import EventPool
    torch, sbb = P.torch, P.sbb
    stream = torch.cuda.current_stream()
    pool = EventPool(max(len(P.calls[M]) for M in M_list))
    recs = []
    for M in M_list:
        for i, call in enumerate(P.calls[M]):
            x, w, y, m, N, K = call
            sbb.qmm_set_launch_events(P.h, *pool.pairs[i])
            rc = P.lib.qmm_run(P.h, x, w, y, M, N, K, ctypes.c_void_p(stream.cuda_stream))
            if rc:
                raise RuntimeError(sbb.qmm_status_string(rc))
        torch.cuda.synchronize()
        for i, (x, w, y, m, N, K) in enumerate(P.calls[M]):
            recs.append((P.kernel_symbol(M, N, K), shape_class(N, K), M, N, K, pool.elapsed_ms(i)))
    pool.close()
    sym, shp = {}, {}
    for s, cls, M, N, K, ms_ in recs:
        us = ms_ * 1e3
        acc.check_roofline(acc.weight_bytes(N, K), us * 1e-6, what="%s M=%d N=%d K=%d" % (s, M, N, K))
        for key, table in ((s, sym), ("%s M=%d" % (cls, M), shp)):
            d = table.setdefault(key, {"launches": 0, "us": 0.0, "bytes": 0, "weight_bytes": 0})
            d["launches"] += 1
            d["us"] += us
            d["bytes"] += acc.call_bytes(M, N, K)
            d["weight_bytes"] += acc.weight_bytes(N, K)
        if seq is not None:
            seq.append({"symbol": s, "shape": cls, "M": M, "N": N, "K": K})
    return sym, shp


def read_profile(name, field="traffic_bytes_per_dispatch"):
    """key -> value of the "field[key]: value" lines of a committed profile
    summary under profiles/, or {} when it is absent or was taken on other
    kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    vals, sha = {}, None
    for line in open(path):
        if line.startswith("kernel_source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif line.startswith(field + "[") and "]:" in line:
            key = line[len(field) + 1:line.index("]:")]
            vals[key] = float(line.split("]:", 1)[1].strip())
    return vals if sha == kernel_source_sha() else {}


def configs_measure(torch, sbb, synth, acc, h, ceiling_gbs=None, reps=4):
    """The single-matrix workloads, each walking distinct device copies so that
    at least 1 GiB streams between two reads of the same bytes (the 256 MB
    last-level cache cannot serve them): per row count, us per call of a
    graph-replayed sequence (launch gaps included), the kernel's own duration
    (event-timed eager launches over the same copies), weight GB/s and % of
    peak for both, and the HBM traffic per call from the committed counter
    profile (profiles/counters_pass_and_configs.txt) with its GB/s."""
    from skinny_bit_block_amd.events import EventPool
    lib = sbb.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    traffic = read_profile("counters_pass_and_configs.txt")
    rows = []
    for name, N, K, Ms, xs in CONFIGS:
        wb = acc.weight_bytes(N, K)
        R = max(3, -(-(1 << 30) // wb))
        base = torch.from_numpy(synth.weights(N, K, tensor=7, seed=SEED).reshape(-1)).cuda()
        copies = [base] + [base.clone() for _ in range(R - 1)]
        pool = EventPool(R)
        for M in Ms:
            x = torch.from_numpy(synth.acts(M, K, tensor=8, seed=SEED, scale=xs)).cuda()
            y = torch.empty((M, N), device="cuda")
            calls = [(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(c.data_ptr()),
                      ctypes.c_void_p(y.data_ptr())) for c in copies]

            def go(spp):
                for c in calls:
                    rc = lib.qmm_run(h, *c, M, N, K, ctypes.c_void_p(spp))
                    if rc:
                        raise RuntimeError(sbb.qmm_status_string(rc))

            go(stream.cuda_stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                go(torch.cuda.current_stream().cuda_stream)
            g.replay()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e-3 / R)
            ts.sort()
            t = ts[len(ts) // 2]
            # the kernel's own duration, eager launches walking the same copies
            for i, c in enumerate(calls):
                sbb.qmm_set_launch_events(h, *pool.pairs[i])
                rc = lib.qmm_run(h, *c, M, N, K, sp)
                if rc:
                    raise RuntimeError(sbb.qmm_status_string(rc))
            torch.cuda.synchronize()
            kd = sorted(pool.elapsed_ms(i) * 1e-3 for i in range(len(calls)))[len(calls) // 2]
            acc.check_roofline(wb, min(ts), what="%s M=%d" % (name, M))
            acc.check_roofline(wb, kd, what="%s M=%d (kernel)" % (name, M))
            p = sbb.qmm_query_plan(h, M, N, K)
            key = "config %s M=%d" % (shape_class(N, K), M)
            row = {"workload": name, "M": M, "us_per_call": round(t * 1e6, 3),
                   "weight_gbs": round(acc.gbs(wb, t), 1), "pct_hbm_peak": round(acc.pct_of(wb, t, 8e12), 2),
                   "kernel_us": round(kd * 1e6, 3), "kernel_weight_gbs": round(acc.gbs(wb, kd), 1),
                   "kernel_pct_hbm_peak": round(acc.pct_of(wb, kd, 8e12), 2),
                   "kernel": sbb.KERNEL_NAMES[p["kernel"]], "waves_per_wg": p["waves_per_wg"],
                   "splits": p["splits"], "wave_splits": p["wave_splits"], "copies": R}
            if ceiling_gbs:
                row["pct_of_read_ceiling"] = round(100 * acc.gbs(wb, t) / ceiling_gbs, 2)
            if key in traffic:
                row["counter_bytes_per_call"] = int(traffic[key])
                row["counter_gbs"] = round(traffic[key] / kd / 1e9, 1)
                row["counter_pct_hbm_peak"] = round(100 * traffic[key] / kd / 8e12, 2)
            rows.append(row)
            log(json.dumps(row))
        pool.close()
        del copies, base
        torch.cuda.empty_cache()
    return rows


def probes_measure(torch, acc):
    """The memory system and launch path on their own (include/qmm_probe.h):
    a read-only 128-bit streaming kernel over 4 GiB (best of a few grid
    shapes), the same kernel reading one lm_head-sized buffer back to back for
    ~100 ms (sustained read), 513 empty kernels in a graph (the launch gap
    between back-to-back launches of a pass), and the shader clock the compute
    units run at (median over workgroups on every CU)."""
    from skinny_bit_block_amd import probe
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = {}
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    best = None
    for grid, block in ((512, 256), (2048, 256), (4096, 512)):
        probe.qmm_probe_read(big.data_ptr(), big.numel(), grid, block, sink.data_ptr(), sp)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            probe.qmm_probe_read(big.data_ptr(), big.numel(), grid, block, sink.data_ptr(), sp)
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        ts.sort()
        gbs = acc.gbs(big.numel(), ts[2])
        if best is None or gbs > best[0]:
            best = (gbs, grid, block)
    out["read_ceiling"] = {"bytes": big.numel(), "gbs": round(best[0], 1),
                           "pct_hbm_peak": round(100 * best[0] / PEAK_GBS, 2),
                           "grid": best[1], "block": best[2]}
    del big
    nb = acc.weight_bytes(151936, 5120)
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    buf.fill_(2)
    reps = 200
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            probe.qmm_probe_read(buf.data_ptr(), nb, 2048, 256, sink.data_ptr(),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3
    out["sustained_read"] = {"bytes_per_read": nb, "reads": reps, "ms": round(t * 1e3, 2),
                             "gbs": round(acc.gbs(nb * reps, t), 1),
                             "pct_hbm_peak": round(acc.pct_of(nb * reps, t, 8e12), 2)}
    del buf, g
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(513):
            probe.qmm_probe_empty(256, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / 513)
    ts.sort()
    out["launch_gap_us"] = round(ts[2], 3)
    del g
    # shader clock: four 64-thread workgroups per CU, each a dependent FMA chain
    # between two readings of the clock counter and the constant-rate counter
    wgs = 1024
    counts = torch.zeros(4 * wgs, dtype=torch.int64, device="cuda")
    khz = probe.qmm_probe_clock(counts.data_ptr(), wgs, 1 << 20, sp)
    torch.cuda.synchronize()
    c = counts.view(wgs, 4).cpu().numpy().astype("float64")
    ghz = sorted((c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]) * khz * 1e-6)
    out["shader_clock_ghz"] = {"median": round(ghz[wgs // 2], 3), "min": round(ghz[0], 3),
                               "max": round(ghz[-1], 3), "workgroups": wgs, "wall_clock_khz": khz}
    del counts
    torch.cuda.empty_cache()
    return out


def cpu_baseline(budget_s, seconds_single=2.0):
    """The oracle as it stands on the host cores. For each matrix shape of the
    pass and each row count of the headline (1, 4, 8, 16), the oracle computes
    rows of one seeded matrix of that shape in chunks for an equal share of
    the budget; its weight GB/s per (shape, M) then gives the time of a whole
    pass (the 513 calls' bytes at those rates), reported as the pass's weight
    GB/s over the four row counts. The single 2048x2048 workload at M = 4 is
    also timed whole on all threads and on one thread."""
    import numpy as np
    import oracle
    import synth
    from skinny_bit_block_amd import accounting as acc
    shapes = [("square", 5120, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408),
              ("lm_head", 151936, 5120)]
    Ms = (1, 4, 8, 16)
    cores = oracle.threads()  # the OpenMP team of the sampled calls
    share = budget_s / (len(shapes) * len(Ms))
    rates, rows_used = {}, {}
    total_s = 0.0
    for cls, N, K in shapes:
        W = synth.weights(min(N, 8192), K, tensor=1 + 6, seed=SEED)  # rows of one matrix
        n_avail = W.shape[0]
        chunk = 1024 if K <= 5120 else 256
        for M in Ms:
            x = synth.acts(M, K, tensor=100000 + K, seed=SEED)
            rows, t0, start = 0, time.time(), 0
            while time.time() - t0 < share:
                idx = np.arange(start, min(n_avail, start + chunk))
                oracle.qmm_rows(x, W, n_avail, K, idx)
                rows += idx.size
                start = 0 if start + chunk >= n_avail else start + chunk
            dt = time.time() - t0
            total_s += dt
            rates[(cls, M)] = acc.weight_bytes(rows, K) / dt
            rows_used["%s M=%d" % (cls, M)] = rows
    pass_s = {M: sum(acc.weight_bytes(N, K) / rates[(shape_class(N, K), M)]
                     for _, N, K in acc.full_pass_shapes()) for M in Ms}
    pass_bytes = acc.full_pass_weight_bytes()
    value = pass_bytes * len(Ms) / sum(pass_s.values()) / 1e9
    # the single projection, whole, all threads and one thread
    N, K, M = 2048, 2048, 4
    W = synth.weights(N, K, tensor=7, seed=SEED)
    x = synth.acts(M, K, tensor=8, seed=SEED)
    single = {}
    for threads in (0, 1):
        n, t0 = 0, time.time()
        while time.time() - t0 < seconds_single:
            oracle.qmm(x, W, N, K, nthreads=threads)
            n += 1
        dt = (time.time() - t0) / n
        total_s += dt * n
        single["all_threads" if threads == 0 else "one_thread"] = {
            "ms_per_call": round(dt * 1e3, 3), "weight_gbs": round(acc.gbs(acc.weight_bytes(N, K), dt), 4)}
    return {"value": round(value, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "fp64 oracle on rows of one seeded matrix of each pass shape (5120x5120, "
                      "34816x5120, 5120x17408, 151936x5120; up to 8192 rows) at M=1/4/8/16, "
                      "%.1f s of wall time on %d threads; value = weight GB/s of a whole pass "
                      "(513 calls' bytes at the sampled per-shape rates) over the four row counts"
                      % (total_s, cores),
            "ms_per_pass": {str(M): round(pass_s[M] * 1e3, 1) for M in Ms},
            "per_shape_gbs": {"%s M=%d" % k: round(v / 1e9, 4) for k, v in sorted(rates.items())},
            "single_2048x2048_m4": single}


def ids_measure(torch, sbb, synth, acc, h, reps=5):
    """Expert-indexed product on gate+up-shaped experts (E = 8, 100 MB each):
    rows spread over distinct experts, each distinct expert streamed once per
    call. Weight bytes = distinct experts x matrix bytes; graph-replayed
    sequences over all experts keep the weights cold. The same bytes through
    one plain call per distinct expert are timed for comparison."""
    import numpy as np
    E, N, K = 8, 34816, 5120
    mb = acc.weight_bytes(N, K)
    dev = torch.device("cuda:0")
    W = torch.empty(E * mb, dtype=torch.uint8, device=dev)
    host = np.empty(mb, dtype=np.uint8)
    for e in range(E):
        synth.weights(N, K, tensor=90000 + e, seed=SEED, out=host.reshape(N, -1))
        W[e * mb:(e + 1) * mb].copy_(torch.from_numpy(host))
    lib = sbb.load()
    out = {}
    stream = torch.cuda.current_stream()
    for M, ids in ((4, [0, 2, 4, 6]), (8, list(range(8))), (16, [m % 8 for m in range(16)])):
        x = torch.from_numpy(synth.acts(M, K, tensor=91000 + M, seed=SEED)).to(dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        idd = torch.tensor(ids, dtype=torch.int32, device=dev)
        distinct = sorted(set(ids))
        groups = [(e, [m for m in range(M) if ids[m] == e]) for e in distinct]
        xs = [(e, x[rows].contiguous(), torch.empty((len(rows), N), dtype=torch.float32, device=dev))
              for e, rows in groups]

        def run_ids(sp):
            rc = lib.qmm_run_ids(h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(W.data_ptr()),
                                 ctypes.c_void_p(idd.data_ptr()), E, ctypes.c_void_p(y.data_ptr()),
                                 M, N, K, sp)
            if rc:
                raise RuntimeError(sbb.qmm_status_string(rc))

        def run_plain(sp):
            for e, xe, ye in xs:
                rc = lib.qmm_run(h, ctypes.c_void_p(xe.data_ptr()),
                                 ctypes.c_void_p(W.data_ptr() + e * mb), ctypes.c_void_p(ye.data_ptr()),
                                 xe.shape[0], N, K, sp)
                if rc:
                    raise RuntimeError(sbb.qmm_status_string(rc))

        res = {}
        for name, fn in (("ids", run_ids), ("plain_per_expert", run_plain)):
            fn(ctypes.c_void_p(stream.cuda_stream))
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / reps * 1e-3
            acc.check_roofline(len(distinct) * mb, t, what="ids %s M=%d" % (name, M))
            res[name] = {"us_per_call": round(t * 1e6, 2),
                         "weight_gbs": round(acc.gbs(len(distinct) * mb, t), 1)}
        out[str(M)] = {"distinct_experts": len(distinct), "weight_bytes": len(distinct) * mb, **res}
    del W
    torch.cuda.empty_cache()
    return {"workload": "expert-indexed product, E=8 experts of 34816x5120 (gate+up shape), "
                        "rows over distinct experts", "per_m": out}


def nvfp4_measure(torch, sbb, synth, acc, h, reps=5):
    """Block-scaled FP4 product on the shapes the pages bench it on (gate+up
    34816x5120 and a 248320-row lm_head, K=5120, at 1 and 7 rows). Weight bytes
    are counted per call (144 per 256 weights); each timed sequence walks
    distinct device copies of the matrix (8 of gate+up, 2 of lm_head) so the
    weights stream from HBM, replayed as a graph."""
    import numpy as np
    out = {}
    stream = torch.cuda.current_stream()
    dev = torch.device("cuda:0")
    for name, N, K, copies in (("gate_up", 34816, 5120, 8), ("lm_head_248320", 248320, 5120, 2)):
        elems, scales = synth.nvfp4(N, K, tensor=92000 + N % 1000, seed=SEED)
        groups = torch.from_numpy(sbb.qmm_nvfp4_repack(elems, scales, N, K).reshape(-1))
        del elems, scales
        Ws = [groups.to(dev) for _ in range(copies)]
        del groups
        wb = acc.weight_bytes(N, K)
        res = {}
        for M in (1, 7):
            x = torch.from_numpy(synth.acts(M, K, tensor=93000 + M, seed=SEED)).to(dev)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)

            def go(sp):
                for W in Ws:
                    rc = sbb.qmm_run_nvfp4_raw(h, x.data_ptr(), W.data_ptr(), 0.5, y.data_ptr(),
                                               M, N, K, sp)
                    if rc:
                        raise RuntimeError(sbb.qmm_status_string(rc))

            go(stream.cuda_stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                go(torch.cuda.current_stream().cuda_stream)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / reps / len(Ws) * 1e-3
            acc.check_roofline(wb, t, what="nvfp4 %s M=%d" % (name, M))
            res[str(M)] = {"us_per_call": round(t * 1e6, 2), "weight_gbs": round(acc.gbs(wb, t), 1),
                           "pct_hbm_peak": round(acc.pct_of(wb, t, 8e12), 2)}
        out[name] = {"N": N, "K": K, "weight_bytes": wb, "per_m": res}
        del Ws
        torch.cuda.empty_cache()
    return {"workload": "block-scaled FP4 (E2M1 elements, E4M3 scale per 16, fp32 tensor scale), "
                        "seeded random codes, 144-byte groups", "shapes": out}


def int4_measure(torch, sbb, synth, acc, h, reps=5):
    """Plain INT4 product (one binary16 scale per 128 columns) on the gate+up
    (34816x5120) and lm_head (151936x5120) shapes at 1 and 7 rows. Streamed
    bytes are the library's 144-byte groups per 256 weights (the layout's own
    size is 132: two scales and 128 code bytes); each timed sequence walks
    distinct device copies (8 of gate+up, 2 of lm_head), replayed as a graph."""
    out = {}
    stream = torch.cuda.current_stream()
    dev = torch.device("cuda:0")
    for name, N, K, copies in (("gate_up", 34816, 5120, 8), ("lm_head", 151936, 5120, 2)):
        codes, scales = synth.int4(N, K, tensor=94000 + N % 1000, seed=SEED)
        groups = torch.from_numpy(sbb.qmm_int4_repack(codes, scales, N, K).reshape(-1))
        del codes, scales
        Ws = [groups.to(dev) for _ in range(copies)]
        del groups
        wb = acc.weight_bytes(N, K)
        res = {}
        for M in (1, 7):
            x = torch.from_numpy(synth.acts(M, K, tensor=95000 + M, seed=SEED)).to(dev)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)

            def go(sp):
                for W in Ws:
                    rc = sbb.qmm_run_int4_raw(h, x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K,
                                              sp)
                    if rc:
                        raise RuntimeError(sbb.qmm_status_string(rc))

            go(stream.cuda_stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                go(torch.cuda.current_stream().cuda_stream)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / reps / len(Ws) * 1e-3
            acc.check_roofline(wb, t, what="int4 %s M=%d" % (name, M))
            res[str(M)] = {"us_per_call": round(t * 1e6, 2), "weight_gbs": round(acc.gbs(wb, t), 1),
                           "pct_hbm_peak": round(acc.pct_of(wb, t, 8e12), 2)}
        out[name] = {"N": N, "K": K, "weight_bytes": wb, "format_bytes": N * K // 256 * 132,
                     "per_m": res}
        del Ws
        torch.cuda.empty_cache()
    return {"workload": "plain INT4 (two's-complement codes, binary16 scale per 128 columns), "
                        "seeded random codes, 144-byte groups", "shapes": out}


GDN_LAYERS, GDN_B, GDN_H, GDN_M, GDN_L, GDN_D = 48, 32, 48, 4, 8, 128


def gdn_flops(n_log, M, H, D=GDN_D):
    """Algorithmic flops of a recurrent-update call: per state element and row,
    s . k (2), the decay and write alpha s + u k (3), and s . q for a new row
    (2); the per-row scalars are not counted."""
    return int(sum(H * D * D * (5 * int(nl) + 7 * M) for nl in n_log))


def gdn_measure(torch, reps=10):
    """The Gated DeltaNet update with log replay (include/gdn.h) on the
    verify pass's recurrent layers: 48 layers, each a call over 32 sequences
    of 48 heads of 128 x 128 fp32 state (3 MiB per sequence and layer, 4.8 GB
    for the 48 layers), 4 new rows per sequence and a log of n_log[b] = b mod 9
    kept rows, all folded into the base state (commit = n_log). A pass is the
    48 calls back to back, replayed as a graph; rates are per call of that
    pass, and events around eager single calls are reported beside them."""
    import numpy as np
    import synth
    from skinny_bit_block_amd import gdn
    B, H, M, L, D = GDN_B, GDN_H, GDN_M, GDN_L, GDN_D
    dev = torch.device("cuda:0")
    base = torch.from_numpy(synth.gdn_state(B, H, D, D, tensor=700, seed=SEED)).to(dev)
    states = [base] + [base.clone() for _ in range(GDN_LAYERS - 1)]
    log = {k: torch.from_numpy(v).to(dev) for k, v in
           synth.gdn_rows(B, L, H, D, D, tensor=701, seed=SEED, queries=False).items()}
    new = {k: torch.from_numpy(v).to(dev) for k, v in synth.gdn_rows(B, M, H, D, D, tensor=702, seed=SEED).items()}
    n_log_h = np.array([b % 9 for b in range(B)], dtype=np.int32)
    n_log = torch.from_numpy(n_log_h).to(dev)
    commit = n_log.clone()
    o = torch.empty((B, M, H, D), device=dev)
    stream = torch.cuda.current_stream()

    def go(sp):
        for st in states:
            gdn.gdn_replay_update(st, log, n_log, new, o, commit=commit, stream=sp)

    go(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.graph(g, stream=side):
        go(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    ts.sort()
    t_pass = ts[len(ts) // 2]
    # kernel durations: events around single eager calls (each call ~tens of us)
    ks = []
    for st in states[:16]:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        gdn.gdn_replay_update(st, log, n_log, new, o, commit=commit, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        ks.append(a.elapsed_time(b) * 1e-3)
    ks.sort()
    t_call = ks[len(ks) // 2]
    nbytes = gdn.gdn_call_bytes(B, M, H, D, D, int(n_log_h.sum()), int((n_log_h > 0).sum()))
    flops = gdn_flops(n_log_h, M, H)
    hbm_s, alu_s = nbytes / 8e12, flops / 157.3e12
    del states, base
    torch.cuda.empty_cache()
    per_call_pass = t_pass / GDN_LAYERS
    hbm_bound = hbm_s >= alu_s
    # the roofline divides by the per-call time inside the graphed pass (launch
    # gaps included: conservative); the committed rocprofv3 trace of
    # `bench.py --mode gdn` gives the kernel's own mean beside it
    prof = {}
    path = os.path.join(ROOT, "profiles", "gdn_replay_kernel_layer_call.md")
    src = os.path.join(ROOT, "skinny_bit_block_amd", "csrc", "gdn_kernels.hip")
    if os.path.exists(path):
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        text = open(path).read()
        if ("gdn_kernels.hip %s" % sha) in text:
            for line in text.splitlines():
                if line.startswith("mean_kernel_us[gdn_replay_kernel]:"):
                    prof["profile_avg_kernel_us"] = float(line.split(":")[1])
                if line.startswith("traffic_bytes_per_dispatch[gdn_replay_kernel]:"):
                    prof["traffic"] = float(line.split(":")[1])
    roof = {"bound": "hbm" if hbm_bound else "alu",
            "achieved": round(nbytes / per_call_pass / 1e9, 1) if hbm_bound else round(flops / per_call_pass / 1e12, 2),
            "peak": 8000.0 if hbm_bound else 157.3,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round((hbm_s if hbm_bound else alu_s) / per_call_pass, 4),
            "traffic": prof.get("traffic"),
            "timing": "per call of a graph-replayed pass of the 48 layer calls (launch gaps included)",
            "floor_us": round(max(hbm_s, alu_s) * 1e6, 3),
            "alu_floor_us_fp32_vector": round(alu_s * 1e6, 3)}
    if "profile_avg_kernel_us" in prof:
        roof["profile_avg_kernel_us"] = prof["profile_avg_kernel_us"]
        roof["frac_from_profile"] = round((hbm_s if hbm_bound else alu_s) / (prof["profile_avg_kernel_us"] * 1e-6), 4)
    return {
        "workload": "Gated DeltaNet recurrent update with log replay: %d layers x %d sequences x %d "
                    "heads of 128x128 fp32 state (3 MiB per sequence and layer), %d new rows, logs of "
                    "b mod 9 kept rows folded into the base state; synthetic states and rows"
                    % (GDN_LAYERS, B, H, M),
        "ms_per_pass_48_layers": round(t_pass * 1e3, 4),
        "us_per_call_in_pass": round(per_call_pass * 1e6, 3),
        "event_us_per_call": round(t_call * 1e6, 3),
        "bytes_per_call": nbytes, "flops_per_call": flops,
        "gbs": round(nbytes / per_call_pass / 1e9, 1),
        "pct_hbm_peak": round(100 * nbytes / per_call_pass / 8e12, 2),
        "tflops": round(flops / per_call_pass / 1e12, 2),
        "roofline": roof,
    }


def pass_record(P, per_m, acc, ceiling=None):
    out = {}
    for M, ms_ in per_m.items():
        r = {"ms_per_pass": round(ms_, 4),
             "weight_gbs": round(acc.gbs(P.weight_bytes, ms_ * 1e-3), 1),
             "pct_hbm_peak": round(acc.pct_of(P.weight_bytes, ms_ * 1e-3, 8e12), 2)}
        if ceiling:
            r["pct_of_read_ceiling"] = round(100 * acc.gbs(P.weight_bytes, ms_ * 1e-3) / ceiling, 2)
        out[str(M)] = r
    return out


def mode_pass(args, torch, sbb, synth, acc):
    ms = [int(v) for v in args.ms.split(",")]
    extra = [int(v) for v in args.extra_ms.split(",") if v and int(v) not in ms]
    P = Pass(torch, sbb, synth, acc, ms + extra, args.layers)
    if not args.no_graph:
        P.capture()
        if not args.no_fused:
            P.capture(fused=True)
        log("graphs captured")
    ms_step, per_m, wall = time_passes(P, args.steps, args.warmup, graph=not args.no_graph, ms=ms)
    log("timed %d steps: %.3f ms/step (wall %.2f s)" % (args.steps, ms_step, wall))
    for M in ms:
        acc.check_roofline(P.weight_bytes, per_m[M] * 1e-3, what="pass M=%d" % M)
    out = {}
    probes = None
    if not args.no_probes:
        log("memory-system probes...")
        probes = probes_measure(torch, acc)
    ceiling = probes["read_ceiling"]["gbs"] if probes else None
    out["per_m"] = pass_record(P, per_m, acc, ceiling)
    x_per_m = {}
    if extra:
        _, x_per_m, _ = time_passes(P, args.steps, args.warmup, graph=not args.no_graph, ms=extra)
        for M in extra:
            acc.check_roofline(P.weight_bytes, x_per_m[M] * 1e-3, what="pass M=%d" % M)
        out["per_m_extra"] = pass_record(P, x_per_m, acc, ceiling)
    if not args.no_fused and not args.no_graph:
        log("fused-projection pass...")
        f_step, f_per_m, _ = time_passes(P, args.steps, args.warmup, graph=True, ms=ms + extra,
                                         fused=True)
        for M in ms + extra:
            acc.check_roofline(P.weight_bytes, f_per_m[M] * 1e-3, what="fused pass M=%d" % M)
        fm = ms
        out["fused_pass"] = {
            "workload": "the same 15.73 GB with each layer's five same-input 5120-wide projections "
                        "as one 25600x5120 call (the sixth, gate+up and down separate): %d calls"
                        % len(P.fused_calls[ms[0]]),
            "weight_gbs": round(acc.gbs(P.weight_bytes * len(fm), sum(f_per_m[M] for M in fm) * 1e-3), 1),
            "per_m": pass_record(P, f_per_m, acc, ceiling)}
    if not args.no_eager and not args.no_graph:
        e_step, e_per_m, _ = time_passes(P, max(3, args.steps // 4), 1, graph=False, ms=ms)
        out["eager"] = {str(M): {"ms_per_pass": round(e_per_m[M], 4),
                                 "weight_gbs": round(acc.gbs(P.weight_bytes, e_per_m[M] * 1e-3), 1)}
                        for M in ms}
    sym, shp = kernel_timing(P, ms)
    dom = max(sym, key=lambda k: sym[k]["us"])
    d = sym[dom]
    avg_s = d["us"] / d["launches"] * 1e-6
    bytes_per_launch = d["bytes"] / d["launches"]
    achieved = bytes_per_launch / avg_s / 1e9
    traffic = read_profile("counters_pass_and_configs.txt").get(dom)
    out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                       "frac": round(achieved / PEAK_GBS, 4),
                       "traffic": None if traffic is None else round(traffic, 0),
                       "kernel": dom, "launches": d["launches"],
                       "avg_kernel_us": round(avg_s * 1e6, 3),
                       "algorithmic_bytes_per_launch": round(bytes_per_launch, 0),
                       "timing": "kernel start to end (HIP events recorded by the launch itself), "
                                 "one eager pass per M in %s" % ms}
    trace_us = read_profile("kernels_trace_pass_and_configs.md", "mean_kernel_us").get(dom)
    if trace_us is not None:
        # the committed rocprofv3 trace of the same launches (bench.py --mode kernels)
        out["roofline"]["profile_avg_kernel_us"] = trace_us
        out["roofline"]["frac_from_profile"] = round(bytes_per_launch / (trace_us * 1e-6) / 1e9 / PEAK_GBS, 4)
    if ceiling:
        out["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling, 4)
    out["kernels"] = {k: {"launches": v["launches"], "avg_us": round(v["us"] / v["launches"], 3),
                          "share": round(v["us"] / sum(w["us"] for w in sym.values()), 4)}
                      for k, v in sorted(sym.items())}
    out["kernel_per_shape"] = {k: {"launches": v["launches"], "avg_us": round(v["us"] / v["launches"], 3),
                                   "weight_gbs": round(v["weight_bytes"] / (v["us"] * 1e-6) / 1e9, 1),
                                   "pct_hbm_peak": round(100 * v["weight_bytes"] / (v["us"] * 1e-6) / 8e12, 2)}
                               for k, v in sorted(shp.items())}
    if probes:
        out["probes"] = probes
    if not args.no_configs:
        log("single-matrix workloads...")
        out["configs"] = configs_measure(torch, sbb, synth, acc, P.h, ceiling)
    if not args.no_ids:
        log("expert-indexed product...")
        out["ids"] = ids_measure(torch, sbb, synth, acc, P.h)
    if not args.no_fp4:
        log("block-scaled FP4 product...")
        out["nvfp4"] = nvfp4_measure(torch, sbb, synth, acc, P.h)
    if not args.no_int4:
        log("plain INT4 product...")
        out["int4"] = int4_measure(torch, sbb, synth, acc, P.h)
    if not args.no_gdn:
        log("recurrent update with log replay...")
        out["gdn"] = gdn_measure(torch)
        log(json.dumps(out["gdn"]))
    value = acc.gbs(P.weight_bytes * len(ms), ms_step * 1e-3)
    prop = torch.cuda.get_device_properties(0)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "full model pass: 64 layers x (6 x 5120x5120 + gate+up 34816x5120 + "
                               "down 5120x17408) + lm_head 151936x5120, Q4_K super-blocks, "
                               "%d matrices, %d weight bytes" % (len(P.shapes), P.weight_bytes),
                   "rows_per_pass": ms, "passes_per_step": len(ms),
                   "timing": "hipGraph replay" if not args.no_graph else "eager",
                   "pct_hbm_peak": round(100 * value / PEAK_GBS, 2),
                   "floor_ms_per_pass": round(P.weight_bytes / 8e12 * 1e3, 4),
                   "device": "%s, %d CUs" % (getattr(prop, "gcnArchName", prop.name),
                                            prop.multi_processor_count)},
    }
    if ceiling:
        line["config"]["pct_of_read_ceiling"] = round(100 * value / ceiling, 2)
    line.update(out)
    line["kernel_source_sha256"] = kernel_source_sha()
    if not args.no_cpu:
        log("cpu baseline (oracle)...")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    sbb.qmm_destroy(P.h)
    print(json.dumps(line), flush=True)


def mode_kernels(args, torch, sbb, synth, acc):
    """Only event-timed eager launches, for rocprofv3 runs: one pass per M,
    then two calls of each single-matrix workload per row count (on two
    distinct copies). --seq-out writes the launch sequence (symbol, shape, M)
    that profile_summary.py maps the profiler's dispatches onto."""
    ms = [int(v) for v in args.ms.split(",")]
    P = Pass(torch, sbb, synth, acc, ms, args.layers)
    from skinny_bit_block_amd.events import EventPool
    seq = []
    for _ in range(max(1, args.steps)):
        sym, shp = kernel_timing(P, ms, seq)
    pool = EventPool(1)
    lib = sbb.load()
    stream = torch.cuda.current_stream()
    for name, N, K, Ms, xs in CONFIGS:
        Ws = [torch.from_numpy(synth.weights(N, K, tensor=7 + i, seed=SEED).reshape(-1)).cuda()
              for i in range(2)]
        for M in Ms:
            x = torch.from_numpy(synth.acts(M, K, tensor=8, seed=SEED, scale=xs)).cuda()
            y = torch.empty((M, N), device="cuda")
            for W in Ws:
                sbb.qmm_set_launch_events(P.h, *pool.pairs[0])
                rc = lib.qmm_run(P.h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(W.data_ptr()),
                                 ctypes.c_void_p(y.data_ptr()), M, N, K, ctypes.c_void_p(stream.cuda_stream))
                if rc:
                    raise RuntimeError(sbb.qmm_status_string(rc))
                seq.append({"symbol": P.kernel_symbol(M, N, K), "shape": "config " + shape_class(N, K),
                            "M": M, "N": N, "K": K})
        torch.cuda.synchronize()
        del Ws
    if args.seq_out:
        json.dump({"kernel_source_sha256": kernel_source_sha(), "launches": seq}, open(args.seq_out, "w"))
    print(json.dumps({k: {"launches": v["launches"], "avg_us": round(v["us"] / v["launches"], 3)}
                      for k, v in sorted(sym.items())}))


SWITCH_SHAPES = [(5120, 5120), (34816, 5120), (5120, 17408), (151936, 5120)]


def mode_switch(args, torch, sbb, synth, acc):
    """Both kernels forced at 1..8 rows on every matrix shape of the pass, for
    rocprofv3 runs that decide the row-vector (VALU dot2) / tiled (MFMA) switch
    point. Each (shape, M, kernel) runs every launch shape the table holds for
    the matrix (its entries from 1 to 16 rows) that fits at M rows, each three
    times on a rotation of distinct copies of the matrix larger than the
    last-level cache (cold weights). --seq-out writes the launch sequence."""
    from skinny_bit_block_amd.events import EventPool
    lib = sbb.load()
    h = sbb.qmm_create(0)
    stream = torch.cuda.current_stream()
    pool = EventPool(1)
    seq, res = [], {}
    for N, K in SWITCH_SHAPES:
        nb = acc.weight_bytes(N, K)
        copies = max(3, -(-(512 << 20) // nb))
        host = synth.weights(N, K, tensor=11, seed=SEED).reshape(-1)
        W = torch.empty(copies * nb, dtype=torch.uint8, device="cuda")
        for c in range(copies):
            W[c * nb:(c + 1) * nb].copy_(torch.from_numpy(host))
        rot = 0
        for M in range(1, 9):
            x = torch.from_numpy(synth.acts(M, K, tensor=12, seed=SEED)).cuda()
            y = torch.empty((M, N), device="cuda")
            for kernel in (sbb.KERNEL_VECTOR, sbb.KERNEL_TILED):
                sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)
                sbb.qmm_set_shape(h, 0, 0, 0)
                sbb.qmm_set_wave_splits(h, 0)
                table_kernel = sbb.KERNEL_NAMES[sbb.qmm_query_plan(h, M, N, K)["kernel"]]
                shapes = []
                for m_src in [M] + list(range(1, 17)):
                    p = sbb.qmm_query_plan(h, m_src, N, K)
                    s = (p["waves_per_wg"], p["splits"], p["wave_splits"])
                    if s not in shapes:
                        shapes.append(s)
                for waves, splits, wsplit in shapes:
                    sbb.qmm_set_kernel(h, kernel)
                    sbb.qmm_set_shape(h, waves, splits, 0)
                    sbb.qmm_set_wave_splits(h, wsplit)
                    try:
                        sbb.qmm_query_plan(h, M, N, K)
                    except sbb.QmmError:
                        continue  # that shape's staged x does not fit at M rows
                    name = "qmm_vector_kernel<%d>" % M if kernel == sbb.KERNEL_VECTOR \
                        else "qmm_tiled_kernel<1, false, 0>"
                    times = []
                    for _ in range(3):
                        Wc = W[(rot % copies) * nb:(rot % copies + 1) * nb]
                        rot += 1
                        sbb.qmm_set_launch_events(h, *pool.pairs[0])
                        rc = lib.qmm_run(h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(Wc.data_ptr()),
                                         ctypes.c_void_p(y.data_ptr()), M, N, K,
                                         ctypes.c_void_p(stream.cuda_stream))
                        if rc:
                            raise RuntimeError(sbb.qmm_status_string(rc))
                        torch.cuda.synchronize()
                        times.append(pool.elapsed_ms(0) * 1e3)
                        seq.append({"symbol": name, "shape": shape_class(N, K), "M": M, "N": N, "K": K,
                                    "kernel": sbb.KERNEL_NAMES[kernel], "table_kernel": table_kernel,
                                    "launch": "%d/%d/%d" % (waves, splits, wsplit)})
                    key = "%s M=%d %s %d/%d/%d" % (shape_class(N, K), M, sbb.KERNEL_NAMES[kernel],
                                                   waves, splits, wsplit)
                    res[key] = round(sum(times) / len(times), 3)
            sbb.qmm_set_kernel(h, sbb.KERNEL_AUTO)
            sbb.qmm_set_shape(h, 0, 0, 0)
            sbb.qmm_set_wave_splits(h, 0)
        del W
        torch.cuda.empty_cache()
    pool.close()
    sbb.qmm_destroy(h)
    if args.seq_out:
        json.dump({"kernel_source_sha256": kernel_source_sha(), "launches": seq}, open(args.seq_out, "w"))
    print(json.dumps({"event_us": res}))


def mode_configs(args, torch, sbb, synth, acc):
    """The single-matrix workloads only."""
    h = sbb.qmm_create(0)
    rows = configs_measure(torch, sbb, synth, acc, h)
    sbb.qmm_destroy(h)
    print(json.dumps({"configs": rows}))


def mode_copy(args, torch):
    """A plain device copy of 1 GiB, five times: the known-size reference that
    scales the FETCH_SIZE / WRITE_SIZE counters."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_dispatch": n, "copy_bytes_written_per_dispatch": n,
                      "dispatches": 5}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the skinny product is built and measured on a single "
              "MI355X; --gpus %d is not supported (the multi-GPU sharding is a design note only)"
              % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mode == "copy":
        return mode_copy(args, torch)
    if args.mode == "gdn":  # the recurrent-update record alone (for profiler runs)
        print(json.dumps(gdn_measure(torch, reps=max(1, args.steps))))
        return
    import synth
    import skinny_bit_block_amd as sbb
    from skinny_bit_block_amd import accounting as acc
    {"pass": mode_pass, "configs": mode_configs, "kernels": mode_kernels,
     "switch": mode_switch}[args.mode](
        args, torch, sbb, synth, acc)


if __name__ == "__main__":
    main()

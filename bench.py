#!/usr/bin/env python3
"""Benchmark of the skinny quantized product on one MI355X.

Default mode (the contract): one step = one full model pass at each of
M = 1, 4, 8, 16 rows. A pass is 513 calls back-to-back on one stream: per layer
(64) six 5120x5120 projections, the fused gate+up (34816x5120) and the down
projection (5120x17408), then the 151936x5120 lm_head: 15,725,813,760 bytes of
4.5-bit super-blocks, every matrix distinct and resident in HBM before timing.
Prints one JSON line: weight GB/s over the step (value), ms per pass per M, the
same for a 32-row pass (per_m_extra, timed separately and not part of value),
the roofline of the dominant kernel measured live with HIP events, and the
oracle timed on the host cores on a bounded sample as a baseline.

Other modes: --mode configs (per-matrix timings of the four single-matrix
workloads with rotating copies), --mode kernels (only the per-launch kernel
timing region, for rocprofv3 runs), --mode copy (a plain device copy of known
size, the calibration of the FETCH_SIZE / WRITE_SIZE counters).
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
KERNEL_SRC = os.path.join(ROOT, "skinny_bit_block_amd", "csrc", "qmm_kernels.hip")


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def kernel_source_sha():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--ms", default="1,4,8,16")
    ap.add_argument("--extra-ms", default="32",
                    help="row counts also timed per pass but not part of value ('' for none)")
    ap.add_argument("--mode", default="pass", choices=["pass", "configs", "kernels", "copy"])
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ids", action="store_true", help="skip the expert-indexed record")
    ap.add_argument("--no-fp4", action="store_true", help="skip the block-scaled FP4 record")
    ap.add_argument("--no-int4", action="store_true", help="skip the plain INT4 record")
    ap.add_argument("--no-eager", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="one allocation per matrix instead of one weight arena")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--layers", type=int, default=64, help="(for quick tests only; the metric needs 64)")
    return ap.parse_args()


class Pass:
    """Device-resident weights, activations and outputs of one full model pass."""

    def __init__(self, torch, sbb, synth, acc, ms, layers, arena=True):
        self.torch, self.sbb = torch, sbb
        self.shapes = [s for s in acc.full_pass_shapes()
                       if s[0] == "lm_head" or int(s[0][1:].split(".")[0]) < layers]
        self.weight_bytes = sum(acc.weight_bytes(N, K) for _, N, K in self.shapes)
        self.ms = ms
        dev = torch.device("cuda:0")
        self.W = []
        bufs = {}
        t0 = time.time()
        # all matrices in one device allocation, each at a 2 MiB-aligned offset
        # (the way an inference engine keeps its weights)
        align = 2 << 20
        offs, total = [], 0
        for _, N, K in self.shapes:
            offs.append(total)
            total += -(-acc.weight_bytes(N, K) // align) * align
        self.arena = torch.empty(total, dtype=torch.uint8, device=dev) if arena else None
        for i, (name, N, K) in enumerate(self.shapes):
            nbytes = acc.weight_bytes(N, K)
            if nbytes not in bufs:
                import numpy as np
                bufs[nbytes] = np.empty(nbytes, dtype=np.uint8)
            host = bufs[nbytes]
            synth.weights(N, K, tensor=i + 1, seed=SEED, out=host.reshape(N, -1))
            if arena:
                d = self.arena[offs[i]:offs[i] + nbytes]
            else:
                d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            d.copy_(torch.from_numpy(host))
            self.W.append(d)
            if i % 64 == 0:
                log("weights %d/%d resident (%.1f s)" % (i + 1, len(self.shapes), time.time() - t0))
        torch.cuda.synchronize()
        log("all %d matrices resident: %.3f GB in %.1f s"
            % (len(self.shapes), self.weight_bytes / 1e9, time.time() - t0))
        self.x = {}
        self.y = {}
        for M in ms:
            for K in sorted({K for _, _, K in self.shapes}):
                xs = synth.acts(M, K, tensor=100000 + K, seed=SEED)
                self.x[(M, K)] = torch.from_numpy(xs).to(dev)
            for N in sorted({N for _, N, _ in self.shapes}):
                self.y[(M, N)] = torch.empty((M, N), dtype=torch.float32, device=dev)
        self.lib = sbb.load()
        self.h = sbb.qmm_create(0)
        self.calls = {}
        for M in ms:
            lst = []
            for (name, N, K), Wd in zip(self.shapes, self.W):
                lst.append((ctypes.c_void_p(self.x[(M, K)].data_ptr()), ctypes.c_void_p(Wd.data_ptr()),
                            ctypes.c_void_p(self.y[(M, N)].data_ptr()), M, N, K))
            self.calls[M] = lst
        self.graphs = {}

    def run(self, M, stream_ptr):
        fn, h = self.lib.qmm_run, self.h
        s = ctypes.c_void_p(stream_ptr)
        for x, w, y, m, n, k in self.calls[M]:
            rc = fn(h, x, w, y, m, n, k, s)
            if rc:
                raise RuntimeError("qmm_run failed: %s" % self.sbb.qmm_status_string(rc))

    def capture(self):
        torch = self.torch
        for M in self.ms:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.run(M, side.cuda_stream)  # warm the kernels outside the capture
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                self.run(M, torch.cuda.current_stream().cuda_stream)
            self.graphs[M] = g
        torch.cuda.synchronize()

    def plan(self, M, N, K):
        return self.sbb.qmm_query_plan(self.h, M, N, K)

    def kernel_symbol(self, M, N, K):
        p = self.plan(M, N, K)
        if p["kernel"] == self.sbb.KERNEL_TILED:
            return "qmm_tiled_kernel<%d, false, 0>" % (1 if M <= 16 else 2)
        return "qmm_vector_kernel<%d>" % M


def time_passes(P, steps, warmup, graph, ms=None):
    """Per-M ms per pass (for the row counts ms, default all of P's), timed with
    HIP events on the stream the kernels run on."""
    torch = P.torch
    stream = torch.cuda.current_stream()
    ms = P.ms if ms is None else ms
    ev = {M: [] for M in ms}

    def one_step(record):
        for M in ms:
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            if graph:
                P.graphs[M].replay()
            else:
                P.run(M, stream.cuda_stream)
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


def kernel_timing(P, M_list):
    """Every launch of one eager pass per M bracketed by HIP events on its stream:
    per-symbol launch count, mean duration and algorithmic bytes per launch."""
    from skinny_bit_block_amd import accounting as acc
    torch = P.torch
    stream = torch.cuda.current_stream()
    recs = []
    for M in M_list:
        for (name, N, K), call in zip(P.shapes, P.calls[M]):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = P.lib.qmm_run(P.h, call[0], call[1], call[2], M, N, K, ctypes.c_void_p(stream.cuda_stream))
            if rc:
                raise RuntimeError(P.sbb.qmm_status_string(rc))
            b.record(stream)
            recs.append((P.kernel_symbol(M, N, K), M, N, K, a, b))
    torch.cuda.synchronize()
    sym = {}
    for s, M, N, K, a, b in recs:
        d = sym.setdefault(s, {"launches": 0, "ms": 0.0, "bytes": 0, "weight_bytes": 0})
        d["launches"] += 1
        d["ms"] += a.elapsed_time(b)
        d["bytes"] += acc.call_bytes(M, N, K)
        d["weight_bytes"] += acc.weight_bytes(N, K)
        acc.check_roofline(acc.weight_bytes(N, K), a.elapsed_time(b) * 1e-3, what="%s M=%d N=%d K=%d" % (s, M, N, K))
    return sym


def read_traffic(symbol):
    """Counter-measured HBM bytes per dispatch of `symbol`, from the committed
    rocprofv3 summary, or None if absent or taken on other kernel source."""
    path = os.path.join(ROOT, "profiles", "counters_full_pass.txt")
    if not os.path.exists(path):
        return None
    sha, val = None, None
    for line in open(path):
        if line.startswith("kernel_source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        if line.startswith("traffic_bytes_per_dispatch[%s]:" % symbol):
            val = float(line.split(":", 1)[1].strip())
    if sha != kernel_source_sha() or val is None:
        return None
    return val


def cpu_baseline(budget_s):
    """The oracle as it stands on the host cores: rows of one gate+up matrix
    (N = 34816, K = 5120) at M = 1, 4, 8, 16, cycling over the matrix in
    chunks until each M has used a quarter of the time budget."""
    import numpy as np
    import oracle
    import synth
    from skinny_bit_block_amd import accounting as acc
    N, K = 34816, 5120
    W = synth.weights(N, K, tensor=1 + 6, seed=SEED)
    per_m = budget_s / 4
    chunk = 4096
    total_bytes, total_s, rows_used = 0, 0.0, {}
    for M in (1, 4, 8, 16):
        x = synth.acts(M, K, tensor=100000 + K, seed=SEED)
        rows, t0, start = 0, time.time(), 0
        while time.time() - t0 < per_m:
            idx = np.arange(start, min(N, start + chunk))
            oracle.qmm_rows(x, W, N, K, idx)
            rows += idx.size
            start = 0 if start + chunk >= N else start + chunk
        dt = time.time() - t0
        total_bytes += acc.weight_bytes(rows, K)
        total_s += dt
        rows_used[M] = rows
    return {"value": round(total_bytes / total_s / 1e9, 4), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "fp64 oracle on rows of one gate+up matrix (N=34816, K=5120), cycled in chunks "
                      "of 4096 rows: %s rows at M=1/4/8/16, %.1f s of wall time on %d threads; "
                      "weight GB/s over the sample"
                      % ("/".join(str(rows_used[m]) for m in (1, 4, 8, 16)), total_s, oracle.threads())}


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


def mode_pass(args, torch, sbb, synth, acc):
    ms = [int(v) for v in args.ms.split(",")]
    extra = [int(v) for v in args.extra_ms.split(",") if v and int(v) not in ms]
    P = Pass(torch, sbb, synth, acc, ms + extra, args.layers, arena=not args.separate)
    if not args.no_graph:
        P.capture()
        log("graphs captured")
    ms_step, per_m, wall = time_passes(P, args.steps, args.warmup, graph=not args.no_graph, ms=ms)
    log("timed %d steps: %.3f ms/step (wall %.2f s)" % (args.steps, ms_step, wall))
    for M in ms:
        acc.check_roofline(P.weight_bytes, per_m[M] * 1e-3, what="pass M=%d" % M)
    out = {}
    out["per_m"] = {str(M): {"ms_per_pass": round(per_m[M], 4),
                             "weight_gbs": round(acc.gbs(P.weight_bytes, per_m[M] * 1e-3), 1),
                             "pct_hbm_peak": round(acc.pct_of(P.weight_bytes, per_m[M] * 1e-3, 8e12), 2)}
                    for M in ms}
    if extra:
        _, x_per_m, _ = time_passes(P, args.steps, args.warmup, graph=not args.no_graph, ms=extra)
        for M in extra:
            acc.check_roofline(P.weight_bytes, x_per_m[M] * 1e-3, what="pass M=%d" % M)
        out["per_m_extra"] = {str(M): {"ms_per_pass": round(x_per_m[M], 4),
                                       "weight_gbs": round(acc.gbs(P.weight_bytes, x_per_m[M] * 1e-3), 1),
                                       "pct_hbm_peak": round(acc.pct_of(P.weight_bytes, x_per_m[M] * 1e-3, 8e12), 2)}
                              for M in extra}
    if not args.no_eager and not args.no_graph:
        e_step, e_per_m, _ = time_passes(P, max(3, args.steps // 4), 1, graph=False, ms=ms)
        out["eager"] = {str(M): {"ms_per_pass": round(e_per_m[M], 4),
                                 "weight_gbs": round(acc.gbs(P.weight_bytes, e_per_m[M] * 1e-3), 1)}
                        for M in ms}
    sym = kernel_timing(P, ms)
    dom = max(sym, key=lambda s: sym[s]["ms"])
    d = sym[dom]
    avg_s = d["ms"] / d["launches"] * 1e-3
    bytes_per_launch = d["bytes"] / d["launches"]
    achieved = bytes_per_launch / avg_s / 1e9
    traffic = read_traffic(dom)
    out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                       "frac": round(achieved / PEAK_GBS, 4),
                       "traffic": None if traffic is None else round(traffic, 0),
                       "kernel": dom, "launches": d["launches"],
                       "avg_launch_us": round(avg_s * 1e6, 3),
                       "algorithmic_bytes_per_launch": round(bytes_per_launch, 0)}
    out["kernels"] = {s: {"launches": v["launches"], "avg_us": round(v["ms"] / v["launches"] * 1e3, 3),
                          "share": round(v["ms"] / sum(w["ms"] for w in sym.values()), 4)}
                      for s, v in sorted(sym.items())}
    if not args.no_ids:
        log("expert-indexed product...")
        out["ids"] = ids_measure(torch, sbb, synth, acc, P.h)
    if not args.no_fp4:
        log("block-scaled FP4 product...")
        out["nvfp4"] = nvfp4_measure(torch, sbb, synth, acc, P.h)
    if not args.no_int4:
        log("plain INT4 product...")
        out["int4"] = int4_measure(torch, sbb, synth, acc, P.h)
    value = acc.gbs(P.weight_bytes * len(ms), ms_step * 1e-3)
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
                   "floor_ms_per_pass": round(P.weight_bytes / 8e12 * 1e3, 4)},
    }
    line.update(out)
    line["kernel_source_sha256"] = kernel_source_sha()
    if not args.no_cpu:
        log("cpu baseline (oracle)...")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    sbb.qmm_destroy(P.h)
    print(json.dumps(line), flush=True)


def mode_kernels(args, torch, sbb, synth, acc):
    """Only the per-launch timing region (one eager pass per M): for rocprofv3."""
    ms = [int(v) for v in args.ms.split(",")]
    P = Pass(torch, sbb, synth, acc, ms, args.layers, arena=not args.separate)
    for _ in range(max(1, args.steps)):
        sym = kernel_timing(P, ms)
    print(json.dumps({s: {"launches": v["launches"], "avg_us": round(v["ms"] / v["launches"] * 1e3, 3),
                          "bytes_per_launch": v["bytes"] / v["launches"]} for s, v in sorted(sym.items())}))


def mode_configs(args, torch, sbb, synth, acc):
    """The single-matrix workloads, rotating distinct copies so that >= 1 GiB is
    streamed between two reads of the same bytes (the 256 MB last-level cache
    cannot serve them)."""
    cfgs = [("single 2048x2048", 2048, 2048, [4], 1.0),
            ("gate+up 34816x5120", 34816, 5120, [1, 2, 4, 7, 8, 9, 16], 1.0),
            ("down 5120x17408", 5120, 17408, [1, 4, 8, 16], 0.1),
            ("lm_head 151936x5120", 151936, 5120, [1, 7], 1.0)]
    h = sbb.qmm_create(0)
    lib = sbb.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    rows = []
    for name, N, K, Ms, xs in cfgs:
        wb = acc.weight_bytes(N, K)
        R = max(3, -(-(1 << 30) // wb))
        base = torch.from_numpy(synth.weights(N, K, tensor=7, seed=SEED).reshape(-1)).cuda()
        copies = [base] + [base.clone() for _ in range(R - 1)]
        for M in Ms:
            x = torch.from_numpy(synth.acts(M, K, tensor=8, seed=SEED, scale=xs)).cuda()
            y = torch.empty((M, N), device="cuda")
            calls = [(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(c.data_ptr()),
                      ctypes.c_void_p(y.data_ptr())) for c in copies]
            n_launch = max(R * 4, int(0.05 / max(wb / 8e12, 1e-7)))
            for i in range(R * 2):
                lib.qmm_run(h, *calls[i % R], M, N, K, sp)
            torch.cuda.synchronize()
            meds = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for i in range(n_launch):
                    lib.qmm_run(h, *calls[i % R], M, N, K, sp)
                b.record(stream)
                torch.cuda.synchronize()
                meds.append(a.elapsed_time(b) / n_launch)
            meds.sort()
            t = meds[2] * 1e-3
            acc.check_roofline(wb, meds[0] * 1e-3, what="%s M=%d" % (name, M))
            p = sbb.qmm_query_plan(h, M, N, K)
            rows.append({"workload": name, "M": M, "us_per_call": round(t * 1e6, 3),
                         "weight_gbs": round(acc.gbs(wb, t), 1),
                         "pct_hbm_peak": round(acc.pct_of(wb, t, 8e12), 2),
                         "kernel": sbb.KERNEL_NAMES[p["kernel"]], "splits": p["splits"],
                         "waves_per_wg": p["waves_per_wg"], "copies": R})
            log(json.dumps(rows[-1]))
        del copies, base
        torch.cuda.empty_cache()
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
    import synth
    import skinny_bit_block_amd as sbb
    from skinny_bit_block_amd import accounting as acc
    {"pass": mode_pass, "configs": mode_configs, "kernels": mode_kernels}[args.mode](
        args, torch, sbb, synth, acc)


if __name__ == "__main__":
    main()

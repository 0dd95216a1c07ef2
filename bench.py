#!/usr/bin/env python
"""Benchmark of the BitDelta hot path on one MI355X; prints ONE JSON line.

Workload of the headline number: the decode layer of the post's 70B-class
model, one 4096 x 4096 bf16 weight with packed 1-bit deltas, through the fused
linear (W_eff never materialised).  One step is one pass of the fused decode
linear over one batch at every decode size:
  m = 1, 4, 16 tokens with per-row alpha, then the same three with the
  per-matrix alpha,
each launch reading its own weight set out of 16 rotating sets (571 MB of
weights, more than the 256 MB MALL, so every launch streams from HBM).
`value` is the step's algorithmic HBM bytes (W_base + packed signs + alpha +
x + y per launch) divided by its time: GB/s.  The steps are captured in HIP
graphs (one per weight set) so the microsecond-scale decode launches are not
bound by host launch overhead; the timed region replays exactly --steps steps.

The same line carries:
  kernels     per-entry average launch time (HIP events around graph
              replays of that entry alone, on its own stream) and GB/s: the
              six fused decode launches, and the offline passes (compress
              with per-row and per-matrix alpha, reconstruct) beside them;
  roofline    for the dominant kernel of the step (largest launch time),
              against 8 TB/s, with its counter-measured HBM traffic;
  rooflines   the same for every decode entry, compress and reconstruct, each
              prefill shape (TFLOP/s against 2.5 PFLOP/s) and the grouped GEMM;
  prefill     the fused MFMA GEMM at m = 2048 tokens on the q/o, k/v,
              gate/up and down shapes, with the oracle on 512 output rows
              (extrapolated) beside it;
  grouped     14 variants over one shared 8192 x 8192 base, 4096 tokens in a
              Zipf(1.1) split (TFLOP/s), with the oracle beside it;
  similarity  K-Merge's cosine similarity of the 14 variants: over the packed
              code and over the full fp32 task vectors W_ft - W_base (GB/s);
  monosoup    the MonoSoup merge of two 8192 x 8192 checkpoints;
  stack       the 70B-shaped stack resident on the GPU (80 layers x 7
              linears, 14 delta sets, 257 GB): compress of one variant,
              512-token prefill and 1-token decode through all 560 linears,
              cold-start upload of one variant's deltas (--no-stack skips it);
  context     reference points from the vendor libraries through torch: a
              34 MiB copy, plain bf16 GEMMs on the prefill shapes, and the
              unfused path (reconstruct to HBM, then a plain GEMM) beside the
              fused call, with the overhead of each over the plain GEMM;
  cpu_baseline  the oracle timed on the host cores on the same decode step,
              at the same shape, on host-generated inputs.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused BitDelta linear: prefill TFLOP/s + decode HBM GB/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

R = C = 4096          # decode layer
DECODE_M = (1, 4, 16)
SETS = 16
PREFILL_SHAPES = [("q/o", 8192, 8192), ("k/v", 1024, 8192), ("gate/up", 28672, 8192), ("down", 8192, 28672)]
PREFILL_M = 2048

# GPU kernels behind each measured decode-layer entry: source file under
# csrc/ and the kernel names (regular expressions on rocprofv3's demangled
# names).  The step is the fused linear entries; compress and reconstruct are
# measured beside it.
STEP_KERNELS = {
    "compress_row": ("compress.hip", [r"compress_rows<true, false>"]),
    "compress_matrix": ("compress.hip", [r"compress_rows<true, true>", r"alpha_matrix_finish"]),
    "reconstruct": ("reconstruct.hip", [r"reconstruct_rows<false>"]),
    "linear_m1_row": ("gemv.hip", [r"gemv_stream<1, 1, \d+, false, true, false>"]),
    "linear_m1_matrix": ("gemv.hip", [r"gemv_stream<1, 1, \d+, true, true, false>"]),
    "linear_m4_row": ("gemv.hip", [r"gemv_stream<4, 1, \d+, false, true, true>"]),
    "linear_m4_matrix": ("gemv.hip", [r"gemv_stream<4, 1, \d+, true, true, true>"]),
    "linear_m16_row": ("gemv.hip", [r"gemv_rows<8, 8, 1, 1, false, false>"]),
    "linear_m16_matrix": ("gemv.hip", [r"gemv_rows<8, 8, 1, 1, false, true>"]),
}
STEP = [f"linear_m{m}_{mode}" for mode in ("row", "matrix") for m in DECODE_M]
OFFLINE = ["compress_row", "compress_matrix", "reconstruct"]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-grouped", action="store_true")
    p.add_argument("--no-monosoup", action="store_true")
    p.add_argument("--summarize-kernels", nargs=3, metavar=("TRACE_CSV", "PATTERN", "ANCHOR"),
                   help="per-kernel totals of the kernels matching PATTERN, per dispatch of ANCHOR")
    p.add_argument("--no-context", action="store_true",
                   help="skip the vendor-library reference points (read stream, plain GEMM)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for cpu_baseline")
    p.add_argument("--kernel-reps", type=int, default=125,
                   help="graph replays per kernel for the per-kernel timings (lower it under a profiler)")
    p.add_argument("--stack", action="store_true",
                   help="instead of the decode-layer line, build the full 70B-shaped stack (80 layers x 7 linears, "
                        "14 delta sets, 257 GB resident) and time a compress pass over one variant's full weight set, "
                        "a 512-token prefill pass and a 1-token decode pass through every linear")
    p.add_argument("--stack-layers", type=int, default=80)
    p.add_argument("--no-stack", action="store_true", help="skip the 70B-shaped stack section of the default line")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the decode step (counter runs of other sections; the line then has no value)")
    p.add_argument("--prefill-shapes", default="", help="comma-separated prefill shapes to run (default: all)")
    p.add_argument("--grouped-rows", type=int, default=8192,
                   help="d_out of the grouped layer (8192; 28672 puts the shared base above the MALL)")
    p.add_argument("--summarize-gemm-counters", nargs=4, metavar=("ENTRY", "FETCH_CSV", "WRITE_CSV", "COPY_MB"),
                   help="record the HBM bytes per call of one prefill shape (fused and unfused) or of the grouped "
                        "GEMM from a counter pass of that section alone into profiles/traffic.json (no GPU)")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="after the run, copy a buffer of this many MiB once (torch copy_), so counter runs can "
                        "calibrate FETCH_SIZE / WRITE_SIZE against a kernel of known traffic")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU: turn the counter_collection CSVs of a FETCH_SIZE run and a WRITE_SIZE run (each "
                        "made with --copy-probe-mb) into HBM bytes per launch of each decode-step kernel; writes "
                        "profiles/traffic.json and prints a table")
    p.add_argument("--summarize-wave-states", nargs=2, metavar=("CSV_A", "CSV_B"),
                   help="wave-state fractions per kernel from the two WAVE_STATE_COUNTERS --pmc runs")
    p.add_argument("--summarize-stack", metavar="TRACE_CSV",
                   help="per-linear decode durations of the 70B-shaped stack from a kernel trace of --stack")
    p.add_argument("--summarize-trace", metavar="TRACE_CSV",
                   help="no GPU: per (kernel, grid) dispatch count and durations from a kernel_trace CSV")
    p.add_argument("--summarize-mfma", metavar="COUNTER_CSV",
                   help="print MFMA busy, clock and VALU/LDS per MFMA of the prefill kernels from a "
                        "rocprofv3 --pmc run of the MFMA counters, and exit")
    p.add_argument("--copy-mb", type=int, default=256, help="--copy-probe-mb of the counter runs")
    p.add_argument("--command", default="", help="command line recorded in profiles/traffic.json")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------- decode step


class DecodeStep:
    """Buffers and the ordered list of C-ABI launches of one step per weight set."""

    def __init__(self, torch, bd, synth):
        self.torch, self.bd = torch, bd
        dev = torch.device("cuda")
        self.sets = []
        for i in range(SETS):
            w_base, w_ft = synth.device_layer(R, C, seed=0, index=i)
            s = dict(w_base=w_base, w_ft=w_ft,
                     signs=torch.empty((R, C // 8), dtype=torch.uint8, device=dev),
                     alpha=torch.empty((R,), dtype=torch.float32, device=dev),
                     alpha_m=torch.empty((1,), dtype=torch.float32, device=dev),
                     ws=torch.empty((bd.lib.bitdelta_compress_workspace(R, C, 1),), dtype=torch.uint8, device=dev))
            self.sets.append(s)
        # every set's code (both alpha modes) exists before the linear launches read it
        for i in range(SETS):
            self.launch("compress_row", i, torch.cuda.current_stream())
            self.launch("compress_matrix", i, torch.cuda.current_stream())
        self.weff = [torch.empty((R, C), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        self.x = {m: synth.device_activations(m, C, seed=0, index=m) for m in DECODE_M}
        self.y = {m: [torch.empty((m, R), dtype=torch.bfloat16, device=dev) for _ in range(2)] for m in DECODE_M}
        torch.cuda.synchronize()
        self.bytes = self.algorithmic_bytes()

    @staticmethod
    def algorithmic_bytes():
        """Entries of the step in order -> algorithmic bytes per launch (inputs
        read once + outputs written once)."""
        w = R * C
        b = {
            "compress_row": w * 2 + w * 4 + w // 8 + 4 * R,
            "compress_matrix": w * 2 + w * 4 + w // 8 + 4,
            "reconstruct": w * 2 + w // 8 + 4 * R + w * 2,
        }
        for m in DECODE_M:
            b[f"linear_m{m}_row"] = w * 2 + w // 8 + 4 * R + 2 * m * C + 2 * m * R
            b[f"linear_m{m}_matrix"] = w * 2 + w // 8 + 4 + 2 * m * C + 2 * m * R
        return b

    def launch(self, name, i, stream):
        """Enqueue one kernel of the step for weight set i on `stream` (raw C ABI)."""
        bd, s = self.bd, self.sets[i]
        P = ctypes.c_void_p
        st = P(stream.cuda_stream)
        if name == "compress_row":
            rc = bd.lib.bitdelta_compress(P(s["w_base"].data_ptr()), P(s["w_ft"].data_ptr()), bd.BD_F32, R, C,
                                          bd.BD_ALPHA_ROW, P(s["signs"].data_ptr()), P(s["alpha"].data_ptr()),
                                          None, 0, st)
        elif name == "compress_matrix":
            rc = bd.lib.bitdelta_compress(P(s["w_base"].data_ptr()), P(s["w_ft"].data_ptr()), bd.BD_F32, R, C,
                                          bd.BD_ALPHA_MATRIX, P(s["signs"].data_ptr()), P(s["alpha_m"].data_ptr()),
                                          P(s["ws"].data_ptr()), s["ws"].numel(), st)
        elif name == "reconstruct":
            rc = bd.lib.bitdelta_reconstruct(P(s["w_base"].data_ptr()), P(s["signs"].data_ptr()),
                                             P(s["alpha"].data_ptr()), bd.BD_ALPHA_ROW, R, C,
                                             P(self.weff[i % 2].data_ptr()), st)
        else:
            _, mm, mode = name.split("_")
            m = int(mm[1:])
            a = s["alpha"] if mode == "row" else s["alpha_m"]
            rc = bd.lib.bitdelta_linear(P(self.x[m].data_ptr()), m, P(s["w_base"].data_ptr()),
                                        P(s["signs"].data_ptr()), P(a.data_ptr()),
                                        bd.BD_ALPHA_ROW if mode == "row" else bd.BD_ALPHA_MATRIX, R, C,
                                        P(self.y[m][i % 2].data_ptr()), None, 0, st)
        bd.check(rc)

    def step(self, i, stream):
        """Step i: its j-th launch uses weight set (len(STEP) * i + j) mod SETS,
        so consecutive launches over the replayed steps walk the 16 sets in
        order and no launch finds its weights still cached (a set comes back
        after 15 other launches, more than the 256 MB MALL holds)."""
        n = len(STEP)
        for j, name in enumerate(STEP):
            self.launch(name, (n * i + j) % SETS, stream)

    @property
    def step_bytes(self):
        return sum(self.bytes[k] for k in STEP)


def capture(torch, fn):
    """Capture fn(stream) into a HIP graph (torch's capture stream is current)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(s)  # eager warm-up call outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return g


def time_graphs(torch, graphs, n, warm):
    """Replay graphs round-robin; time exactly n replays with HIP events on the replay stream."""
    stream = torch.cuda.current_stream()
    for k in range(warm):
        graphs[k % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(n):
        graphs[k % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall  # seconds (device events), seconds (host wall)


def run_decode(torch, bd, synth, steps, warmup, kernel_reps):
    ds = DecodeStep(torch, bd, synth)
    step_graphs = [capture(torch, lambda s, i=i: ds.step(i, s)) for i in range(SETS)]
    dev_s, wall_s = time_graphs(torch, step_graphs, steps, warmup)
    # per-kernel: a graph of SETS launches (one per weight set) of that kernel alone
    kernels = {}
    for name, nbytes in ds.bytes.items():
        g = capture(torch, lambda s, name=name: [ds.launch(name, i, s) for i in range(SETS)])
        # 5 repeats of reps / 5 replays: "us" is the average launch over all of
        # them, next to the median and the min of the 5 repeat averages
        reps = max(5, kernel_reps) // 5
        rep_us = []
        for r in range(5):
            t, _ = time_graphs(torch, [g], reps, 4 if r == 0 else 1)
            rep_us.append(t / (reps * SETS) * 1e6)
        us = sum(rep_us) / 5
        kernels[name] = {"us": round(us, 3), "us_median5": round(statistics.median(rep_us), 3),
                         "us_min5": round(min(rep_us), 3), "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1),
                         "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        del g
    del step_graphs
    return ds, dev_s, wall_s, kernels


# -------------------------------------------------------------------- prefill


def prefill_shapes(only):
    """The prefill shapes to run: all, or the comma-separated labels in `only`."""
    want = [w for w in only.split(",") if w]
    return [s for s in PREFILL_SHAPES if not want or s[0] in want]


def run_prefill(torch, bd, synth, reps=10, only=""):
    out = {}
    dev = torch.device("cuda")
    for label, N, K in prefill_shapes(only):
        sets = []
        for i in range(2):
            w_base, w_ft = synth.device_layer(N, K, seed=1, index=10 * i + len(out))
            signs, alpha = bd.compress(w_base, w_ft)
            del w_ft
            sets.append((w_base, signs, alpha))
        x = synth.device_activations(PREFILL_M, K, seed=1, index=len(out))
        y = torch.empty((PREFILL_M, N), dtype=torch.bfloat16, device=dev)
        nws = bd.lib.bitdelta_linear_workspace(PREFILL_M, N, K)
        ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev)
        P = ctypes.c_void_p

        def call(i, s):
            w, sg, a = sets[i % 2]
            bd.check(bd.lib.bitdelta_linear(P(x.data_ptr()), PREFILL_M, P(w.data_ptr()), P(sg.data_ptr()),
                                            P(a.data_ptr()), bd.BD_ALPHA_ROW, N, K, P(y.data_ptr()),
                                            P(ws.data_ptr()), nws, P(s.cuda_stream)))

        stream = torch.cuda.current_stream()
        for i in range(3):
            call(i, stream)
        torch.cuda.synchronize()
        rep_us = []
        for r in range(5):  # 5 repeats of reps calls
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                call(i, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            rep_us.append(e0.elapsed_time(e1) / reps * 1e3)
        us = sum(rep_us) / 5
        flop = 2 * PREFILL_M * N * K
        tf = flop / us / 1e6
        plan = bd.lib.bitdelta_linear_workspace(PREFILL_M, N, K)
        out[label] = {"d_out": N, "d_in": K, "m": PREFILL_M, "us": round(us, 1),
                      "us_median5": round(statistics.median(rep_us), 1), "us_min5": round(min(rep_us), 1),
                      "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
                      "roofline": {"kernel": f"prefill_{label}",
                                   "gpu_kernel": "gemm_tiles_w8" + (" + splitk_reduce" if plan else ""),
                                   "bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                   "traffic": traffic_record(f"prefill_{label}"), "flop_per_launch": flop,
                                   "avg_launch_us": round(us, 1)}}
        log(f"prefill {label} [{N},{K}] m={PREFILL_M}: {us:.1f} us, {tf:.1f} TFLOP/s")
        del sets, x, y
        torch.cuda.empty_cache()
    tot_flop = sum(2.0 * PREFILL_M * v["d_out"] * v["d_in"] for v in out.values())
    tot_us = sum(v["us"] for v in out.values())
    agg = tot_flop / tot_us / 1e6
    return {"shapes": out, "layer_TFLOP/s": round(agg, 1), "layer_frac_mfma": round(agg / BF16_PEAK_TFLOPS, 4),
            "peak_TFLOP/s": BF16_PEAK_TFLOPS}


# -------------------------------------------------------------------- grouped


def run_grouped(torch, bd, synth, reps=10, rows=8192):
    dev = torch.device("cuda")
    N, K = rows, 8192
    V, M = 14, 4096
    w_base = synth.device_normal((N, K), 0.02, 2, synth.tag(synth.TAG_WBASE), dev, torch.bfloat16)
    bv = synth.variant_scales(V, seed=0)
    signs = torch.empty((V, N, K // 8), dtype=torch.uint8, device=dev)
    alpha = torch.empty((V, N), dtype=torch.float32, device=dev)
    w_fts = torch.empty((V, N, K), dtype=torch.float32, device=dev)  # the variants' fp32 weights (3.76 GB)
    for v in range(V):
        w_fts[v].copy_(w_base.float().add_(synth.device_laplace((N, K), float(bv[v]), 2,
                                                                 synth.tag(synth.TAG_VARIANT + v), dev)))
        sg, a = bd.compress(w_base, w_fts[v])
        signs[v].copy_(sg)
        alpha[v].copy_(a)
        del sg, a
    counts = synth.zipf_counts(M, V, 1.1)
    ids = torch.from_numpy(synth.variant_ids(counts, seed=0)).to(dev)
    x = synth.device_activations(M, K, seed=2)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    nws = bd.lib.bitdelta_linear_grouped_workspace(M, V, N, K)
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    P = ctypes.c_void_p
    stream = torch.cuda.current_stream()

    def call():
        bd.check(bd.lib.bitdelta_linear_grouped(P(x.data_ptr()), M, P(ids.data_ptr()), V, P(w_base.data_ptr()),
                                                P(signs.data_ptr()), P(alpha.data_ptr()), bd.BD_ALPHA_ROW, N, K,
                                                P(y.data_ptr()), P(ws.data_ptr()), nws, P(stream.cuda_stream)))

    def timed():
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    # shuffled (the workload) and pre-sorted ids, alternated twice; the best of each
    ids_shuffled = ids
    ids_sorted = torch.sort(ids_shuffled).values.contiguous()
    us = us_sorted = float("inf")
    for _ in range(2):
        ids = ids_shuffled
        us = min(us, timed())
        ids = ids_sorted
        us_sorted = min(us_sorted, timed())
    flop = 2 * M * N * K
    tf = flop / us / 1e6
    log(f"grouped 14 variants [{N},{K}] m=4096: {us:.1f} us, {tf:.1f} TFLOP/s "
        f"(ids pre-sorted: {us_sorted:.1f} us)")
    sim = run_similarity(torch, bd, signs, alpha)
    sim["full_task_vectors"] = run_similarity_delta(torch, bd, w_base, w_fts)
    del w_fts
    torch.cuda.empty_cache()
    roof = {"kernel": "grouped", "gpu_kernel": "bucket_tokens + gemm_tiles_w8 (gathered)", "bound": "mfma",
            "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_record("grouped" if rows == 8192 else f"grouped_{rows}"), "flop_per_launch": flop,
            "avg_launch_us": round(us, 1)}
    return {"d_out": N, "d_in": K, "m": M, "variants": V, "group_sizes": counts, "us": round(us, 1),
            "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
            "us_ids_presorted": round(us_sorted, 1), "roofline": roof}, sim


def run_similarity_delta(torch, bd, w_base, w_fts, reps=5):
    """K-Merge similarity over the full task vectors (W_ft - W_base) of the
    grouped layer's 14 variants: reads the fp32 W_ft of every variant and the
    bf16 base once (algorithmic bytes), writes the two V x V fp64 outputs."""
    V, N, K = w_fts.shape
    dev = w_fts.device
    gram = torch.empty((V, V), dtype=torch.float64, device=dev)
    cos = torch.empty((V, V), dtype=torch.float64, device=dev)
    nws = bd.lib.bitdelta_similarity_delta_workspace(V, N, K)
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    P = ctypes.c_void_p
    stream = torch.cuda.current_stream()

    def call():
        bd.check(bd.lib.bitdelta_similarity_delta(P(w_base.data_ptr()), P(w_fts.data_ptr()), bd.BD_F32, V, N, K,
                                                  P(gram.data_ptr()), P(cos.data_ptr()), P(ws.data_ptr()), nws,
                                                  P(stream.cuda_stream)))

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    rep_us = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        rep_us.append(e0.elapsed_time(e1) / reps * 1e3)
    us = sum(rep_us) / 3
    nbytes = V * N * K * 4 + N * K * 2 + 2 * V * V * 8
    gbs = nbytes / us / 1e3
    log(f"similarity over full task vectors, {V} variants [{N},{K}] fp32: {us:.1f} us, {gbs:.1f} GB/s "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM)")
    return {"variants": V, "d_out": N, "d_in": K, "w_ft": "fp32", "us": round(us, 1),
            "us_min3": round(min(rep_us), 1), "bytes": nbytes, "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def run_similarity(torch, bd, signs, alpha, reps=20):
    """K-Merge similarity (Gram matrix and cosines of the variants' task
    vectors) over the grouped layer's 14 packed sign sets.  Algorithmic bytes:
    the packed signs, alpha and the two V x V fp64 outputs; the int32 counts
    it passes between its two kernels are scratch."""
    V, N, G = signs.shape
    K = 8 * G
    dev = signs.device
    gram = torch.empty((V, V), dtype=torch.float64, device=dev)
    cos = torch.empty((V, V), dtype=torch.float64, device=dev)
    nws = bd.lib.bitdelta_similarity_workspace(V, N, K)
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    P = ctypes.c_void_p
    stream = torch.cuda.current_stream()

    def call():
        bd.check(bd.lib.bitdelta_similarity(P(signs.data_ptr()), P(alpha.data_ptr()), bd.BD_ALPHA_ROW, V, N, K,
                                            P(gram.data_ptr()), P(cos.data_ptr()), P(ws.data_ptr()), nws,
                                            P(stream.cuda_stream)))

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    rep_us = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        rep_us.append(e0.elapsed_time(e1) / reps * 1e3)
    us = sum(rep_us) / 5
    nbytes = V * N * G + V * N * 4 + 2 * V * V * 8
    gbs = nbytes / us / 1e3
    log(f"similarity {V} variants [{N},{K}]: {us:.1f} us, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM)")
    return {"variants": V, "d_out": N, "d_in": K, "us": round(us, 2), "us_median5": round(statistics.median(rep_us), 2),
            "us_min5": round(min(rep_us), 2), "bytes": nbytes, "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


# ---------------------------------------------------------------- monosoup

MS_SHAPE = (8192, 8192)
MS_K, MS_RANK, MS_POWER = 2, 32, 1


def run_monosoup(torch, bd, synth, reps=3):
    """MonoSoup merge (section "MonoSoup"): the current and the best earlier
    checkpoint (k = 2) of an 8192 x 8192 matrix merged through their rank-32
    truncations, one power iteration, sketch of 64 columns; task vectors of
    rank 32 (entry RMS 1e-3) plus N(0, 1e-5^2) noise.  Each Delta pass reads
    both checkpoints (fp32) and the base (bf16): 6 bytes and 2 * 64 flops per
    weight and checkpoint; 2 + 2 * power_iters passes, then the merge reads
    the base and writes fp32 (6 bytes per weight, 2 * k * rp flops)."""
    R, C = MS_SHAPE
    k, r, q = MS_K, MS_RANK, MS_POWER
    dev = torch.device("cuda")
    wb, wf = synth.device_checkpoints(R, C, k, r, 1e-5, seed=5)
    om = synth.device_normal((C, bd.MONOSOUP_SKETCH), 1.0, 5, synth.tag(synth.TAG_OMEGA), dev)
    out = torch.empty((R, C), dtype=torch.float32, device=dev)
    sig = torch.empty((k, r), dtype=torch.float64, device=dev)
    nws = bd.lib.bitdelta_monosoup_workspace(R, C, k, r)
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    P = ctypes.c_void_p
    stream = torch.cuda.current_stream()

    def call():
        bd.check(bd.lib.bitdelta_monosoup(P(wb.data_ptr()), P(wf.data_ptr()), P(om.data_ptr()), k, R, C, r, q,
                                          P(out.data_ptr()), P(sig.data_ptr()), P(ws.data_ptr()), nws,
                                          P(stream.cuda_stream)))

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    rep_us = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        rep_us.append(e0.elapsed_time(e1) / reps * 1e3)
    us = sum(rep_us) / 5
    passes = 2 + 2 * q
    rp = (r + 15) // 16 * 16
    pass_flops = 2.0 * R * C * bd.MONOSOUP_SKETCH * k
    flops = passes * pass_flops + 2.0 * R * C * k * rp
    nbytes = passes * R * C * k * 6 + R * C * 6
    log(f"monosoup k={k} [{R},{C}] rank {r}, {q} power iteration(s): {us / 1e3:.3f} ms per merge, "
        f"{flops / us / 1e6:.1f} TFLOP/s, {nbytes / us / 1e3:.1f} GB/s over {passes} passes + merge")
    res = {"k": k, "rows": R, "cols": C, "rank": r, "power_iters": q, "sketch": bd.MONOSOUP_SKETCH,
           "us": round(us, 1), "us_median5": round(statistics.median(rep_us), 1), "us_min5": round(min(rep_us), 1),
           "passes": passes, "flops": flops, "bytes": nbytes, "TFLOP/s": round(flops / us / 1e6, 1),
           "GB/s": round(nbytes / us / 1e3, 1)}
    del wb, wf, om, out, ws
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------- context


def run_context(torch, reps=20, only=""):
    """Reference points measured with the vendor libraries through torch (not
    the product path): a copy over 16 rotating buffers the size of the decode
    layer's weights (torch copy_, read + write), and a plain bf16 GEMM without
    deltas (torch.mm -> hipBLASLt) on the four prefill shapes at m = 2048,
    weights ~ N(0, 0.02) as in the workload."""
    dev = torch.device("cuda")
    out = {}
    n = (34 << 20) // 2
    src = [torch.randn(n, device=dev, dtype=torch.bfloat16) for _ in range(16)]
    dst = torch.empty_like(src[0])
    for i in range(16):
        dst.copy_(src[i])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(4 * reps):
        dst.copy_(src[i % 16])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (4 * reps) * 1e3
    out["copy_34MiB"] = {"us": round(us, 2), "GB/s": round(4 * n / us / 1e3, 1),
                         "frac_hbm": round(4 * n / us / 1e3 / HBM_PEAK_GBS, 4), "kernel": "torch copy_ (read + write)"}
    log(f"context: copy of 34 MiB (torch copy_, read + write) {us:.2f} us, {4 * n / us / 1e3:.1f} GB/s")
    del src, dst
    gemm = {}
    for label, N, K in prefill_shapes(only):
        # the workload's laws: x ~ N(0, 1), weights ~ N(0, 0.02) (the GEMM's
        # speed depends on the data: its power draw sets the clock)
        x = torch.randn((PREFILL_M, K), device=dev, dtype=torch.bfloat16)
        ws = [(torch.randn((N, K), device=dev) * 0.02).to(torch.bfloat16) for _ in range(2)]
        y = torch.empty((PREFILL_M, N), device=dev, dtype=torch.bfloat16)
        # a longer warm-up than the fused kernel needs: the first few dozen
        # calls of the vendor GEMM run up to 20% slower
        for i in range(40):
            torch.mm(x, ws[i % 2].t(), out=y)
        torch.cuda.synchronize()
        rep_us = []
        for r in range(5):
            e0.record()
            for i in range(reps):
                torch.mm(x, ws[i % 2].t(), out=y)
            e1.record()
            torch.cuda.synchronize()
            rep_us.append(e0.elapsed_time(e1) / reps * 1e3)
        us = sum(rep_us) / 5
        tf = 2.0 * PREFILL_M * N * K / us / 1e6
        gemm[label] = {"us": round(us, 1), "us_median5": round(statistics.median(rep_us), 1),
                       "us_min5": round(min(rep_us), 1), "TFLOP/s": round(tf, 1)}
        log(f"context: plain bf16 GEMM (torch.mm) {label} [{N},{K}] m={PREFILL_M}: {us:.1f} us, {tf:.1f} TFLOP/s")
        del x, ws, y
    out["plain_gemm_m2048"] = gemm
    return out


def run_probes(torch, bd, reps=125):
    """The library's measurement probes (no part of the method): the
    practical streaming-read rate, on 16 rotating buffers of the decode
    layer's weight size (34 MiB, 544 MiB in all, over the MALL) launched back
    to back from a HIP graph like the decode kernels, and on one 1 GiB
    buffer; and the dense bf16 MFMA rate of back-to-back register-operand
    MFMAs on every CU (2 waves per SIMD); and the LDS read, write and
    direct-copy rates per CU."""
    dev = torch.device("cuda")
    P = ctypes.c_void_p
    out = {}
    n = 34 << 20
    bufs = [torch.empty(n // 4, dtype=torch.int32, device=dev).random_() for _ in range(SETS)]
    sink = torch.empty((bd.lib.bitdelta_probe_read_sink_words(n),), dtype=torch.int32, device=dev)

    def launches(s):
        for i in range(reps):
            bd.check(bd.lib.bitdelta_probe_read(P(bufs[i % SETS].data_ptr()), n, P(sink.data_ptr()),
                                                P(s.cuda_stream)))

    g = capture(torch, launches)
    rep_us = [time_graphs(torch, [g], 1, 1)[0] / reps * 1e6 for _ in range(5)]
    us = sum(rep_us) / 5
    out["read_34MiB"] = {"us": round(us, 3), "us_min5": round(min(rep_us), 3), "GB/s": round(n / us / 1e3, 1),
                         "frac_hbm": round(n / us / 1e3 / HBM_PEAK_GBS, 4),
                         "kernel": "probe_read (1 KB per load instruction, 16 rotating buffers, graph-launched)"}
    log(f"context: read probe 34 MiB: {us:.2f} us, {n / us / 1e3:.1f} GB/s")
    del g, bufs, sink
    big = 1 << 30
    buf = torch.empty(big // 4 - 4, dtype=torch.int32, device=dev).random_()   # below 2 GiB, a multiple of 16 B
    nb = buf.numel() * 4
    sink = torch.empty((bd.lib.bitdelta_probe_read_sink_words(nb),), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    call = lambda: bd.check(bd.lib.bitdelta_probe_read(P(buf.data_ptr()), nb, P(sink.data_ptr()),
                                                       P(stream.cuda_stream)))
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 10 * 1e3
    out["read_1GiB"] = {"us": round(us, 1), "GB/s": round(nb / us / 1e3, 1),
                        "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4), "kernel": "probe_read"}
    log(f"context: read probe 1 GiB: {us:.1f} us, {nb / us / 1e3:.1f} GB/s")
    del buf, sink
    blocks, iters = 2 * 256, 4000
    sink = torch.empty((4 * blocks,), dtype=torch.float32, device=dev)
    call = lambda: bd.check(bd.lib.bitdelta_probe_mfma(blocks, iters, 1.0, 1.0, P(sink.data_ptr()),
                                                       P(stream.cuda_stream)))
    call()
    torch.cuda.synchronize()
    rep_us = []
    for _ in range(5):
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        rep_us.append(e0.elapsed_time(e1) * 1e3)
    us = sum(rep_us) / 5
    flop = blocks * 4 * iters * 8 * 32768
    out["mfma_bf16"] = {"us": round(us, 1), "TFLOP/s": round(flop / us / 1e6, 1),
                        "frac_mfma": round(flop / us / 1e6 / BF16_PEAK_TFLOPS, 4), "flop": flop,
                        "kernel": "probe_mfma (v_mfma_f32_32x32x16_bf16 on registers, 2 waves per SIMD)"}
    log(f"context: MFMA probe: {flop / us / 1e6:.1f} TFLOP/s bf16 dense ({us:.1f} us)")
    del sink
    # LDS: one 16-wave workgroup per CU, every wave moving conflict-free
    # contiguous blocks (reads of 16 / 8 bytes per lane, writes of 16, and
    # direct-to-LDS copies of 16 from a 1 MiB L2-resident buffer); the rate
    # per CU is each workgroup's bytes over its own shader-clock cycles
    # (median over the workgroups), the whole-chip rate from the events
    src = torch.empty((1 << 20) // 4, dtype=torch.int32, device=dev).random_()
    blocks, iters = 256, 2048
    lds = {}
    for mode, name, unit in ((0, "read_b128", 1024), (1, "read_b64", 512), (2, "write_b128", 1024),
                             (3, "copy_to_lds", 1024)):
        sink, cycles = bd.probe_lds(blocks, 8, mode, 17, src if mode == 3 else None)
        torch.cuda.synchronize()
        e0.record(stream)
        sink, cycles = bd.probe_lds(blocks, iters, mode, 17, src if mode == 3 else None)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        per_wg = 16 * iters * 8 * unit
        cyc = float(cycles.cpu().double().median())
        lds[name] = {"B/clk per CU": round(per_wg / cyc, 1), "TB/s": round(per_wg * blocks / us / 1e6, 2),
                     "us": round(us, 1)}
        log(f"context: LDS probe {name}: {per_wg / cyc:.1f} B/clock per CU, {per_wg * blocks / us / 1e6:.2f} TB/s")
    out["lds"] = dict(lds, kernel="probe_lds (16 waves, one workgroup per CU, conflict-free blocks; clock "
                                  "cycles from the shader clock counter)")
    return out


def run_unfused(torch, bd, synth, fused, reps=10, only=""):
    """The unfused alternative on the four prefill shapes at m = 2048:
    bitdelta_reconstruct writes W_eff to HBM, then a plain bf16 GEMM
    (torch.mm -> hipBLASLt) reads it; timed back to back per call, next to
    each part alone and the fused call of the same run (`fused`: run_prefill's
    shapes).  Overheads are over the plain GEMM (the same GEMM on W_base, no
    deltas).  Weight-side HBM bytes per weight: fused 2 + 1/8 (W_base + signs);
    unfused 2 + 1/8 + 2 + 2 (+ the W_eff write and its read by the GEMM)."""
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    out = {}

    def timed(fn):
        for i in range(20):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    for label, N, K in prefill_shapes(only):
        sets = []
        for i in range(2):
            w_base, w_ft = synth.device_layer(N, K, seed=1, index=10 * i + len(out))
            signs, alpha = bd.compress(w_base, w_ft)
            del w_ft
            sets.append((w_base, signs, alpha, torch.empty_like(w_base)))
        x = synth.device_activations(PREFILL_M, K, seed=1, index=len(out))
        y = torch.empty((PREFILL_M, N), dtype=torch.bfloat16, device=dev)
        P = ctypes.c_void_p

        def recon(i):
            w, sg, a, we = sets[i % 2]
            bd.check(bd.lib.bitdelta_reconstruct(P(w.data_ptr()), P(sg.data_ptr()), P(a.data_ptr()), bd.BD_ALPHA_ROW,
                                                 N, K, P(we.data_ptr()), P(stream.cuda_stream)))

        def mm(i):
            torch.mm(x, sets[i % 2][3].t(), out=y)

        def both(i):
            recon(i)
            mm(i)

        t_r, t_m, t_u = timed(recon), timed(mm), timed(both)
        t_f = fused["shapes"][label]["us"]
        out[label] = {"reconstruct_us": round(t_r, 1), "plain_gemm_us": round(t_m, 1),
                      "unfused_us": round(t_u, 1), "fused_us": t_f,
                      "fused_overhead_us": round(t_f - t_m, 1), "unfused_overhead_us": round(t_u - t_m, 1),
                      "weight_bytes_fused": N * K * 2 + N * K // 8,
                      "weight_bytes_unfused": N * K * 2 + N * K // 8 + 2 * (N * K * 2)}
        log(f"unfused {label} [{N},{K}] m={PREFILL_M}: reconstruct {t_r:.1f} us, plain GEMM {t_m:.1f} us (each "
            f"alone), the two back to back {t_u:.1f} us; fused {t_f:.1f} us (overhead over the plain GEMM: fused "
            f"{t_f - t_m:+.1f} us, unfused {t_u - t_m:+.1f} us)")
        del sets, x, y
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- 70B stack


def run_stack(torch, bd, synth, n_layers):
    from tenant_fine_tune_amd.stack import LinearStack

    dev = torch.device("cuda")
    free0, total = torch.cuda.mem_get_info()
    t0 = time.perf_counter()
    st = LinearStack(n_layers=n_layers, n_variants=14)
    st.reserve(512)
    log(f"stack: {n_layers} layers x {len(st.shapes)} linears, 14 delta sets, "
        f"{st.resident_bytes() / 1e9:.2f} GB resident (device had {free0 / 1e9:.1f} of {total / 1e9:.1f} GB free)")
    names = [s[0] for s in st.shapes]
    bv = synth.variant_scales(14, seed=4)
    for l, name, d_out, d_in in st.matrices():
        idx = 5000 + 10 * l + names.index(name)
        st.base[l, name].copy_(synth.device_normal((d_out, d_in), 0.02, 4, synth.tag(synth.TAG_WBASE, idx), dev,
                                                   torch.bfloat16))
        g = torch.Generator(device=dev)
        g.manual_seed(idx)
        for v in range(1, 14):  # the other variants: random packed signs, alpha near b_v
            st.signs[v, l, name].copy_(torch.randint(0, 256, st.signs[v, l, name].shape, generator=g, device=dev,
                                                     dtype=torch.int32).to(torch.uint8))
            st.alpha[v, l, name].copy_(torch.rand(st.alpha[v, l, name].shape, generator=g, device=dev)
                                       .mul_(float(bv[v])).add_(float(bv[v]) * 0.5))
        if name == names[-1] and l % 10 == 9:
            torch.cuda.synchronize()
            log(f"stack: layer {l + 1}/{n_layers} filled ({time.perf_counter() - t0:.1f} s)")
    torch.cuda.synchronize()
    log(f"stack: filled in {time.perf_counter() - t0:.1f} s")

    # compress pass over variant 0's full weight set, W_ft streamed one matrix at a time
    stream = torch.cuda.current_stream()
    ev = []

    def make_w_ft(l, name, base):
        idx = 5000 + 10 * l + names.index(name)
        w_ft = base.float().add_(synth.device_laplace(base.shape, float(bv[0]), 4, synth.tag(synth.TAG_DELTA, idx), dev))
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ev.append([e0, None])
        return w_ft

    def after(l, name):
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(stream)
        ev[-1][1] = e1

    st.compress_variant(0, make_w_ft, on_matrix=after)
    torch.cuda.synchronize()
    comp_ms = sum(a.elapsed_time(b) for a, b in ev)
    comp_bytes = sum(d_out * d_in * (2 + 4) + d_out * d_in // 8 + 4 * d_out for _, _, d_out, d_in in st.matrices())
    log(f"stack compress (variant 0, fp32 W_ft): {comp_ms:.1f} ms, {comp_bytes / comp_ms / 1e6:.1f} GB/s")

    out = {"resident_GB": round(st.resident_bytes() / 1e9, 2), "layers": n_layers, "variants": 14,
           "params": st.params(),
           "compress": {"ms": round(comp_ms, 2), "bytes": comp_bytes, "GB/s": round(comp_bytes / comp_ms / 1e6, 1),
                        "frac_hbm": round(comp_bytes / comp_ms / 1e6 / HBM_PEAK_GBS, 4)}}
    widths = {name: d_in for name, _, d_in in st.shapes}
    outs = {name: d_out for name, d_out, _ in st.shapes}
    for label, m, reps in (("prefill", 512, 3), ("decode", 1, 10), ("decode_m4", 4, 10), ("decode_m16", 16, 10)):
        xs = {name: synth.device_activations(m, widths[name], seed=4, index=m + i) for i, name in enumerate(widths)}
        ys = {name: torch.empty((m, outs[name]), dtype=torch.bfloat16, device=dev) for name in outs}
        g = capture(torch, lambda s: st.forward(0, xs, ys, s))
        dev_s, _ = time_graphs(torch, [g], reps, 1)
        ms = dev_s / reps * 1e3
        flop, nbytes = st.flops(m), st.linear_bytes(m)
        out[label] = {"m": m, "ms": round(ms, 3), "TFLOP/s": round(flop / ms / 1e9, 1),
                      "frac_mfma": round(flop / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                      "GB/s": round(nbytes / ms / 1e6, 1), "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                      "bytes": nbytes, "linears": n_layers * len(st.shapes)}
        log(f"stack {label} m={m} through {n_layers * len(st.shapes)} linears: {ms:.2f} ms, "
            f"{flop / ms / 1e9:.1f} TFLOP/s, {nbytes / ms / 1e6:.1f} GB/s")
        del g, xs, ys
    out["delta_upload"] = run_delta_upload(torch, bd, st)
    return out


def run_delta_upload(torch, bd, st, reps=3):
    """Cold start of a variant: its packed deltas for the whole stack (signs +
    alpha of every matrix) copied from pinned host memory to HBM by the
    library's delta-cache loader (bitdelta_cache_host_loader), timed on the
    host around the call (the loader synchronises its stream)."""
    nbytes = sum(d_out * d_in // 8 + 4 * d_out for _, _, d_out, d_in in st.matrices())
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    class HostLoader(ctypes.Structure):
        _fields_ = [("host_ptrs", ctypes.c_void_p), ("stream", ctypes.c_void_p)]

    table = (ctypes.c_void_p * 1)(host.data_ptr())
    hl = HostLoader(ctypes.cast(table, ctypes.c_void_p), torch.cuda.current_stream().cuda_stream)
    ms = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rc = bd.lib.bitdelta_cache_host_loader(ctypes.byref(hl), 0, ctypes.c_void_p(dst.data_ptr()), nbytes)
        ms.append((time.perf_counter() - t0) * 1e3)
        if rc != 0:
            raise RuntimeError(f"host loader failed ({rc})")
    best = min(ms)
    log(f"stack delta upload (one variant, {nbytes / 1e9:.3f} GB, pinned host -> HBM): {best:.1f} ms, "
        f"{nbytes / best / 1e6:.1f} GB/s (the post: about 200 ms for 8.75 GB from NVMe)")
    del host, dst
    return {"bytes": nbytes, "ms_best": round(best, 2), "ms_mean": round(sum(ms) / len(ms), 2),
            "GB/s": round(nbytes / best / 1e6, 1)}


# ----------------------------------------------------------------- cpu oracle


def run_cpu_baseline(target_s):
    """The oracle, untuned, on the same decode step (the fused linear at m = 1,
    4, 16 with per-row and per-matrix alpha) on host-generated inputs of the
    same shape; repeated until about target_s seconds have elapsed."""
    import oracle
    import synth

    w_base, w_ft = synth.layer(R, C, seed=0)
    signs, alpha = oracle.compress(w_base, w_ft)
    _, alpha_m = oracle.compress(w_base, w_ft, per_matrix=True)
    xs = {m: synth.activations(m, C, seed=0, index=m) for m in DECODE_M}
    bytes_step = sum(DecodeStep.algorithmic_bytes()[k] for k in STEP)
    n = 0
    t0 = time.perf_counter()
    while True:
        for m in DECODE_M:
            oracle.linear(xs[m], w_base, signs, alpha)
        for m in DECODE_M:
            oracle.linear(xs[m], w_base, signs, alpha_m, per_matrix=True)
        n += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    gbs = bytes_step * n / el / 1e9
    # the same step on one thread (one step, or more up to a quarter of the budget)
    threads = int(oracle.num_threads())
    oracle.set_num_threads(1)
    try:
        n1 = 0
        t0 = time.perf_counter()
        while True:
            for m in DECODE_M:
                oracle.linear(xs[m], w_base, signs, alpha)
            for m in DECODE_M:
                oracle.linear(xs[m], w_base, signs, alpha_m, per_matrix=True)
            n1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= target_s / 4:
                break
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the full decode step (fused linear m=1,4,16 x 2 alpha modes) on one 4096x4096 layer, "
                      f"host-generated inputs, repeated {n} times in {el:.1f} s",
            "seconds_per_step": round(el / n, 4), "host_cpus": os.cpu_count(),
            "single_thread": {"value": round(bytes_step * n1 / el1 / 1e9, 3), "unit": "GB/s",
                              "seconds_per_step": round(el1 / n1, 4), "steps": n1}}


CPU_ROWS = 512  # output rows of each large matrix the oracle computes; its time is scaled to all rows


def _host_code(rows, d_in, seed, tg, n_variants=None):
    """Host inputs for a timing sample of the oracle: bf16 W_base rows, random
    packed signs and alpha near 1e-3 (the oracle's time does not depend on the
    values)."""
    import numpy as np

    import synth

    wb = synth.to_bf16_bits(synth.normal_f32((rows, d_in), 0.02, seed, tg))
    shape = (rows,) if n_variants is None else (n_variants, rows)
    sg = synth.u64(shape + (d_in // 8,), seed, tg + 1).astype(np.uint8)
    al = (np.abs(synth.normal_f32(shape, 1e-3, seed, tg + 2)) + np.float32(1e-5)).astype(np.float32)
    return wb, sg, al


def run_cpu_prefill():
    """The oracle on the prefill layer (m = 2048 on the q/o, k/v, gate/up, down
    shapes): the first 512 output rows of each, timed once, scaled by d_out /
    512 (extrapolated)."""
    import oracle
    import synth

    out, tot_flop, tot_s = {}, 0.0, 0.0
    for i, (label, N, K) in enumerate(PREFILL_SHAPES):
        wb, sg, al = _host_code(CPU_ROWS, K, 7, 8100 + 10 * i)
        x = synth.activations(PREFILL_M, K, seed=7, index=i)
        t0 = time.perf_counter()
        oracle.linear(x, wb, sg, al)
        el = (time.perf_counter() - t0) * N / CPU_ROWS
        flop = 2.0 * PREFILL_M * N * K
        out[label] = {"seconds_extrapolated": round(el, 2), "TFLOP/s": round(flop / el / 1e12, 5)}
        tot_flop, tot_s = tot_flop + flop, tot_s + el
        log(f"cpu oracle prefill {label}: {el:.1f} s (extrapolated from {CPU_ROWS} rows)")
    return {"kind": "oracle", "cores": int(oracle.num_threads()), "shapes": out,
            "layer_TFLOP/s": round(tot_flop / tot_s / 1e12, 5),
            "sample": f"the first {CPU_ROWS} output rows of each shape at m={PREFILL_M}, host-generated inputs, "
                      f"timed once and scaled by d_out/{CPU_ROWS} (extrapolated)"}


def run_cpu_stack(n_layers):
    """The oracle on the 70B-shaped stack, extrapolated: one layer's seven
    linears at m = 512 (prefill) and m = 1 (decode) and the compress of each
    of its seven matrices from fp32 W_ft, on the first CPU_ROWS output rows of
    each, scaled by d_out / CPU_ROWS and by the layer count (a host-generated
    stack would take about 411 GB of inputs)."""
    import oracle
    import synth
    from tenant_fine_tune_amd.stack import LAYER_SHAPES

    pre = dec = comp = 0.0
    for i, (name, d_out, d_in) in enumerate(LAYER_SHAPES):
        w_base, w_ft = synth.layer(CPU_ROWS, d_in, seed=9, index=9300 + i)
        t0 = time.perf_counter()
        sg, al = oracle.compress(w_base, w_ft)
        comp += (time.perf_counter() - t0) * d_out / CPU_ROWS
        for m, acc in ((512, "pre"), (1, "dec")):
            x = synth.activations(m, d_in, seed=9, index=9400 + 10 * i + m % 7)
            t0 = time.perf_counter()
            oracle.linear(x, w_base, sg, al)
            el = (time.perf_counter() - t0) * d_out / CPU_ROWS
            if acc == "pre":
                pre += el
            else:
                dec += el
    out = {"kind": "oracle", "cores": int(oracle.num_threads()),
           "prefill_m512_s": round(pre * n_layers, 1), "decode_m1_s": round(dec * n_layers, 2),
           "compress_variant_s": round(comp * n_layers, 1),
           "sample": f"one layer's 7 linears and their compress on the first {CPU_ROWS} output rows, "
                     f"host-generated inputs, scaled by d_out/{CPU_ROWS} and x {n_layers} layers (extrapolated)"}
    log(f"cpu oracle stack ({n_layers} layers, extrapolated): prefill m=512 {out['prefill_m512_s']} s, "
        f"decode m=1 {out['decode_m1_s']} s, compress of a variant {out['compress_variant_s']} s")
    return out


def run_cpu_grouped(counts):
    """The oracle on the grouped layer (14 variants, 4096 tokens, Zipf split):
    the first 512 output rows, timed once, scaled by 8192 / 512."""
    import oracle
    import synth

    N = K = 8192
    V, M = len(counts), sum(counts)
    wb, sg, al = _host_code(CPU_ROWS, K, 8, 8200, n_variants=V)
    ids = synth.variant_ids(counts, seed=0)
    x = synth.activations(M, K, seed=8)
    t0 = time.perf_counter()
    oracle.linear_grouped(x, ids, wb, sg, al)
    el = (time.perf_counter() - t0) * N / CPU_ROWS
    flop = 2.0 * M * N * K
    log(f"cpu oracle grouped: {el:.1f} s (extrapolated from {CPU_ROWS} rows)")
    return {"kind": "oracle", "cores": int(oracle.num_threads()), "seconds_extrapolated": round(el, 2),
            "TFLOP/s": round(flop / el / 1e12, 5),
            "sample": f"the first {CPU_ROWS} output rows of the shared 8192x8192 layer, 14 variants, {M} tokens, "
                      f"host-generated inputs, timed once and scaled by {N}/{CPU_ROWS} (extrapolated)"}


# ----------------------------------------------------------------------- main


def hbm_roofline(entry, k):
    """Roofline record of a decode-layer entry: algorithmic bytes per launch
    over its average launch time, against 8 TB/s, with the counter-measured
    HBM bytes per launch (null when the counters predate its source)."""
    return {"kernel": entry, "gpu_kernel": STEP_KERNELS[entry][1][0], "bound": "hbm", "achieved": k["GB/s"],
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k["GB/s"] / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(entry), "algorithmic_bytes_per_launch": k["bytes"], "avg_launch_us": k["us"]}


def traffic_record(entry):
    """HBM bytes per launch of a prefill shape or the grouped GEMM from the
    committed counter runs (profiles/traffic.json), if taken on the current
    gemm.hip; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    e = rec.get("gemm", {}).get(entry)
    if not e or e.get("source_sha") != source_sha("gemm.hip"):
        return None
    return e.get("bytes_per_launch")


def traffic_for(entry):
    """HBM bytes per launch of a decode-step entry from the committed counter
    runs (profiles/traffic.json), if they were taken on the current source of
    its kernels; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    e = rec.get("kernels", {}).get(entry)
    if not e or e.get("source_sha") != source_sha(STEP_KERNELS[entry][0]):
        return None
    return e.get("bytes_per_launch")


def _code_only(text):
    """Source text without its comments and blank lines (a comment edit does
    not change a kernel, so it does not retire the counter runs)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_sha(src):
    """Hash of the code of a kernel source file and the device headers it
    includes (comments left out)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tenant_fine_tune_amd", "csrc")
    for f in (src, "bd_device.h", "bd_launch.h"):
        h.update(_code_only(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def _short(name):
    import re

    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name)


def _copy_probe(dispatches):
    """Counter value of the copy probe: the run's last copy-kernel dispatch
    (bench.py --copy-probe-mb issues it after everything else; earlier copies
    of other sizes, e.g. torch's copy_ of a whole weight tensor, are not it)."""
    vals = [v for n, v in dispatches if "copyBuffer" in n]
    if not vals:
        raise SystemExit("no copy-kernel dispatch in the counter CSV: run with --copy-probe-mb")
    return vals[-1]


def summarize_counters(fetch_csv, write_csv, copy_mb, command, out_dir=None):
    """Scale the per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of each decode-step
    kernel by what the same counters read for a copy of copy_mb MiB, and
    record HBM bytes per launch next to the algorithmic bytes (traffic.json
    in out_dir, by default profiles/)."""
    import csv
    import re
    import statistics

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        return [(_short(r["Kernel_Name"]), int(r["Grid_Size"]), float(r["Counter_Value"]) * 1024.0) for r in rows]

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mb << 20
    cf = _copy_probe([(n, v) for n, _, v in fetch])
    cw = _copy_probe([(n, v) for n, _, v in write])
    f_fetch, f_write = copy_bytes / cf, copy_bytes / cw
    algo = DecodeStep.algorithmic_bytes()
    out = {"command": command, "calibration": {"copy_bytes": copy_bytes, "fetch_factor": round(f_fetch, 4),
                                               "write_factor": round(f_write, 4)}, "kernels": {}}
    lines = [f"calibration: a {copy_mb} MiB copy reads FETCH_SIZE x {f_fetch:.4f} and WRITE_SIZE x {f_write:.4f}",
             f"{'entry':18s} {'kernel':46s} {'n':>4s} {'fetch B':>12s} {'write B':>12s} {'HBM B':>12s} "
             f"{'algorithmic B':>13s} {'ratio':>6s}"]
    for entry, (src, pats) in STEP_KERNELS.items():
        tf = tw = 0.0
        names, n = [], 0
        for pat in pats:
            rx = re.compile(pat)
            # the decode step's dispatches: the grid seen most often (other
            # calls of the same kernel, e.g. the grouped run's compresses,
            # have other grids)
            grids = [g for nm, g, _ in fetch if rx.search(nm)]
            grid = max(set(grids), key=grids.count) if grids else None
            fv = [v for nm, g, v in fetch if rx.search(nm) and g == grid]
            wv = [v for nm, g, v in write if rx.search(nm) and g == grid]
            if not fv or not wv:
                raise SystemExit(f"no dispatches of {pat} in the counter CSVs")
            tf += statistics.median(fv) * f_fetch
            tw += statistics.median(wv) * f_write
            names.append(next(nm for nm, _, _ in fetch if rx.search(nm)))
            n = len(fv)
        total = tf + tw
        out["kernels"][entry] = {"kernels": names, "source": src, "source_sha": source_sha(src),
                                 "fetch_bytes": round(tf), "write_bytes": round(tw), "bytes_per_launch": round(total),
                                 "algorithmic_bytes": algo[entry], "ratio": round(total / algo[entry], 4)}
        lines.append(f"{entry:18s} {' + '.join(names)[:46]:46s} {n:4d} {tf:12.0f} {tw:12.0f} {total:12.0f} "
                     f"{algo[entry]:13d} {total / algo[entry]:6.3f}")
    # grouped layer (14 variants sharing one 8192 x 8192 W_base, 4096 tokens), if in the runs
    rx = re.compile(r"gemm_tiles_w8<false, true, false, \d+>")
    fv = [v for nm, _, v in fetch if rx.search(nm)]
    wv = [v for nm, _, v in write if rx.search(nm)]
    if fv and wv:
        n_ = k_ = 8192
        tf_, tw_ = statistics.median(fv) * f_fetch, statistics.median(wv) * f_write
        w_bytes, s_bytes, x_bytes = n_ * k_ * 2, 14 * n_ * k_ // 8, 4096 * k_ * 2
        out["grouped"] = {"kernel": "gemm_tiles_w8<false, true, false, 256>", "fetch_bytes": round(tf_),
                          "write_bytes": round(tw_), "w_base_bytes": w_bytes, "signs_bytes": s_bytes,
                          "x_bytes": x_bytes, "fetch_over_w_base": round(tf_ / w_bytes, 3)}
        lines.append(f"grouped GEMM (14 variants, 4096 tokens): fetched {tf_:.0f} B, written {tw_:.0f} B per launch; "
                     f"W_base {w_bytes} B, all 14 sign sets {s_bytes} B, x {x_bytes} B; fetched / W_base = "
                     f"{tf_ / w_bytes:.3f} (a launch per variant would fetch W_base 14 times)")
    # MonoSoup (k = 2 checkpoints of 8192 x 8192, rank 32), if in the runs: the Delta passes read
    # 6 B per weight and checkpoint (fp32 W_i + bf16 W_base); the merge reads W_base and writes fp32
    R_, C_ = MS_SHAPE
    ms = {"ms_pass<false>": MS_K * R_ * C_ * 6, "ms_pass<true>": MS_K * R_ * C_ * 6, "ms_merge": R_ * C_ * 6}
    for kern, algo_b in ms.items():
        rx = re.compile(re.escape(kern))
        fv = [v for nm, _, v in fetch if rx.search(nm)]
        wv = [v for nm, _, v in write if rx.search(nm)]
        if not fv or not wv:
            continue
        tf_, tw_ = statistics.median(fv) * f_fetch, statistics.median(wv) * f_write
        out.setdefault("monosoup", {})[kern] = {"fetch_bytes": round(tf_), "write_bytes": round(tw_),
                                                "algorithmic_bytes": algo_b,
                                                "ratio": round((tf_ + tw_) / algo_b, 4)}
        lines.append(f"monosoup {kern:16s} fetched {tf_:.0f} B, written {tw_:.0f} B per launch; algorithmic "
                     f"{algo_b} B (6 B per weight{' and checkpoint' if 'pass' in kern else ''}); ratio "
                     f"{(tf_ + tw_) / algo_b:.3f}")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    prev = os.path.join(out_dir, "traffic.json")
    if os.path.exists(prev):  # keep the per-shape GEMM passes recorded beside the decode entries
        try:
            g = json.load(open(prev)).get("gemm")
        except ValueError:
            g = None
        if g:
            out["gemm"] = g
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("\n".join(lines))


def summarize_gemm_counters(entry, fetch_csv, write_csv, copy_mb, command, out_dir=None):
    """HBM bytes per call of one prefill shape or of the grouped GEMM, from a
    FETCH_SIZE and a WRITE_SIZE pass of that section alone (bench.py
    --no-decode --prefill-shapes LABEL, or --no-prefill --grouped-rows N),
    each scaled like the decode entries by a copy of copy_mb MiB.  A call of
    the fused linear is its GEMM launch(es) and, when it splits K, the
    fixed-order reduce; the unfused path (same run, context leg) is the
    reconstruct to HBM plus the vendor GEMM.  Recorded under "gemm" in
    traffic.json with the algorithmic bytes beside it."""
    import csv
    import re
    import statistics

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        return [(_short(r["Kernel_Name"]), float(r["Counter_Value"]) * 1024.0) for r in rows]

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mb << 20
    f_fetch = copy_bytes / _copy_probe(fetch)
    f_write = copy_bytes / _copy_probe(write)

    def per_call(patterns):
        """Sum over the kernels of one call of the median scaled bytes of each;
        the kernels found (a pattern without dispatches adds nothing)."""
        tf = tw = 0.0
        found = []
        for pat in patterns:
            rx = re.compile(pat)
            fv = [v for nm, v in fetch if rx.search(nm)]
            wv = [v for nm, v in write if rx.search(nm)]
            if fv and wv:
                tf += statistics.median(fv) * f_fetch
                tw += statistics.median(wv) * f_write
                found.append(next(nm for nm, _ in fetch if rx.search(nm)))
        return {"kernels": found, "fetch_bytes": round(tf), "write_bytes": round(tw),
                "bytes_per_launch": round(tf + tw)}

    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    gemm = rec.setdefault("gemm", {})
    if entry.startswith("prefill_"):
        label = entry[len("prefill_"):]
        N, K = next((n, k) for lb, n, k in PREFILL_SHAPES if lb == label)
        fused = per_call([r"gemm_tiles_w8<(true|false), false, false, \d+>",
                          r"gemm_tiles_w8<(true|false), false, true, \d+>",
                          r"splitk_reduce"])
        unfused = per_call([r"reconstruct_rows<false>", r"^Cijk|^void Cijk|Cijk_"])
        algo = {"weights_fused": N * K * 2 + N * K // 8 + 4 * N,
                "weights_unfused": N * K * 2 + N * K // 8 + 4 * N + 2 * (N * K * 2),
                "x": PREFILL_M * K * 2, "y": PREFILL_M * N * 2}
        e = {"fused": fused, "unfused": unfused, "algorithmic": algo,
             "bytes_per_launch": fused["bytes_per_launch"], "source_sha": source_sha("gemm.hip"),
             "command": command, "calibration": {"fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)}}
        print(f"{entry}: fused call {fused['fetch_bytes']} B fetched + {fused['write_bytes']} B written "
              f"({' + '.join(fused['kernels'])}); unfused call {unfused['fetch_bytes']} B + {unfused['write_bytes']} B "
              f"({' + '.join(unfused['kernels'])}); weights {algo['weights_fused']} B fused vs "
              f"{algo['weights_unfused']} B unfused algorithmic")
    else:
        rows = int(entry.split("_")[-1]) if entry.startswith("grouped_") else 8192
        g = per_call([r"gemm_tiles_w8<(true|false), true, false, \d+>", r"bucket_tokens"])
        K, V, M = 8192, 14, 4096
        algo = {"w_base": rows * K * 2, "signs": V * rows * K // 8, "alpha": V * rows * 4, "x": M * K * 2,
                "y": M * rows * 2}
        e = {**g, "algorithmic": algo, "algorithmic_bytes": sum(algo.values()),
             "fetch_over_w_base": round(g["fetch_bytes"] / algo["w_base"], 3),
             "fetch_over_reads": round(g["fetch_bytes"] / (algo["w_base"] + algo["signs"] + algo["alpha"] + algo["x"]),
                                       3),
             "source_sha": source_sha("gemm.hip"), "command": command}
        print(f"{entry}: {g['fetch_bytes']} B fetched, {g['write_bytes']} B written per launch; reads algorithmic "
              f"{algo['w_base'] + algo['signs'] + algo['alpha'] + algo['x']} B (W_base {algo['w_base']}): fetched "
              f"{e['fetch_over_reads']}x the reads, {e['fetch_over_w_base']}x W_base")
    gemm[entry] = e
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def summarize_trace(trace_csv, gap=12):
    """Durations (us) of the library kernels from a kernel_trace CSV, per run
    of one (kernel, grid): a run ends when more than `gap` other dispatches
    pass before the next one (so two shapes with one grid stay apart)."""
    import csv
    import statistics

    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    runs, open_run = [], {}  # runs: [key, first dispatch, durations]; open_run: key -> (last dispatch, run)
    for r in rows:
        if "bd::" not in r["Kernel_Name"]:
            continue
        k = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1),
             int(r["Workgroup_Size_X"]))
        i = int(r["Dispatch_Id"])
        if k in open_run and i - open_run[k][0] <= gap:
            j = open_run[k][1]
        else:
            runs.append([k, i, []])
            j = len(runs) - 1
        runs[j][2].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
        open_run[k] = (i, j)
    print(f"{'kernel':52s} {'threads':>9s} {'wg':>5s} {'first':>7s} {'n':>6s} {'avg us':>9s} {'median':>9s} {'min':>9s}")
    for k, i, v in runs:
        if len(v) < 2:
            continue
        print(f"{k[0][:52]:52s} {k[1]:9d} {k[2]:5d} {i:7d} {len(v):6d} {statistics.mean(v):9.2f} "
              f"{statistics.median(v):9.2f} {min(v):9.2f}")


def summarize_kernels(trace_csv, pattern, anchor):
    """Per-kernel totals for the library kernels whose name contains
    `pattern` (e.g. the MonoSoup kernels, "ms_"): dispatches, average /
    median / min duration, and the time per call of the entry point, taking
    the number of `anchor` dispatches as the number of calls."""
    import csv
    import re

    per = {}
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"]
        if "bd::" not in name or pattern not in name:
            continue
        m = re.search(r"(\w+(<[^>]*>)?)\(", name.replace("(anonymous namespace)::", ""))
        key = m.group(1) if m else _short(name)
        per.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    calls = len(per.get(anchor, [])) or 1
    print(f"{calls} calls (dispatches of {anchor})")
    print(f"{'kernel':28s} {'n':>6s} {'avg us':>9s} {'median':>9s} {'min':>9s} {'us/call':>9s}")
    total = 0.0
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        total += sum(v) / calls
        print(f"{k[:28]:28s} {len(v):6d} {statistics.mean(v):9.2f} {statistics.median(v):9.2f} {min(v):9.2f} "
              f"{sum(v) / calls:9.1f}")
    print(f"{'total':28s} {'':6s} {'':9s} {'':9s} {'':9s} {total:9.1f}")


def summarize_stack(trace_csv, n_layers=80):
    """Decode pass of the 70B-shaped stack from a kernel trace of bench.py
    --stack: the m = 1 launches (gemv_stream<1, ...>) come in the stack's
    order, q, k, v, o, gate, up, down per layer, so dispatch i of them is the
    linear i mod 7.  Per linear shape: launches, average / median duration
    and the rate over its algorithmic bytes (W_base 2 B + signs 1/8 B per
    weight, alpha, x, y); then the whole pass (kernel time only, no gaps).
    The prefill (m = 512) kernels are listed per (kernel, grid)."""
    import csv
    import re

    from tenant_fine_tune_amd.stack import LAYER_SHAPES

    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
    dec = [r for r in rows if re.search(r"gemv_stream<1, ", r["Kernel_Name"])]
    per_pass = n_layers * len(LAYER_SHAPES)
    if not dec or len(dec) % per_pass:
        raise SystemExit(f"{len(dec)} m = 1 launches: not whole passes of {per_pass} linears")
    passes = len(dec) // per_pass
    print(f"decode m = 1: {passes} passes x {per_pass} linears")
    print(f"{'linear':8s} {'d_out':>6s} {'d_in':>6s} {'kernel':40s} {'n':>6s} {'avg us':>8s} {'median':>8s} "
          f"{'bytes':>11s} {'GB/s':>7s}")
    tot_us = tot_b = 0.0
    for j, (name, d_out, d_in) in enumerate(LAYER_SHAPES):
        sel = dec[j::len(LAYER_SHAPES)]
        v = [dur(r) for r in sel]
        b = d_out * d_in * 2 + d_out * d_in // 8 + 4 * d_out + 2 * d_in + 2 * d_out
        avg = statistics.mean(v)
        tot_us += sum(v)
        tot_b += b * len(v)
        print(f"{name:8s} {d_out:6d} {d_in:6d} {_short(sel[0]['Kernel_Name'])[:40]:40s} {len(v):6d} {avg:8.2f} "
              f"{statistics.median(v):8.2f} {b:11d} {b / avg / 1e3:7.1f}")
    print(f"pass: {tot_us / passes / 1e3:.3f} ms of kernel time for {tot_b / passes / 1e9:.2f} GB: "
          f"{tot_b / tot_us / 1e3:.1f} GB/s ({tot_b / tot_us / 1e3 / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s)")
    # the m = 4 and m = 16 passes: one call per linear, in the same order; a
    # call on few long rows is the whole-row kernel plus gemv_split_reduce
    calls = []
    for r in rows:
        name = r["Kernel_Name"]
        if re.search(r"gemv_rows|gemv_stream<[2-4], ", name):
            calls.append([_short(name), dur(r)])
        elif "gemv_split_reduce" in name and calls:
            calls[-1][0] += " + reduce"
            calls[-1][1] += dur(r)
    if calls and len(calls) % per_pass == 0:
        by_m = {4: [], 16: []}
        for p0 in range(0, len(calls), per_pass):
            by_m[4 if "gemv_stream" in calls[p0][0] else 16].extend(calls[p0:p0 + per_pass])
        for m, cs in by_m.items():
            if not cs:
                continue
            passes_m = len(cs) // per_pass
            print(f"decode m = {m}: {passes_m} passes x {per_pass} linears")
            print(f"{'linear':8s} {'d_out':>6s} {'d_in':>6s} {'kernel':40s} {'n':>6s} {'avg us':>8s} {'median':>8s} "
                  f"{'bytes':>11s} {'GB/s':>7s}")
            t_us = t_b = 0.0
            for j, (name, d_out, d_in) in enumerate(LAYER_SHAPES):
                sel = cs[j::len(LAYER_SHAPES)]
                v = [c[1] for c in sel]
                b = d_out * d_in * 2 + d_out * d_in // 8 + 4 * d_out + 2 * m * d_in + 2 * m * d_out
                avg = statistics.mean(v)
                t_us += sum(v)
                t_b += b * len(v)
                print(f"{name:8s} {d_out:6d} {d_in:6d} {sel[0][0][:40]:40s} {len(v):6d} {avg:8.2f} "
                      f"{statistics.median(v):8.2f} {b:11d} {b / avg / 1e3:7.1f}")
            print(f"pass: {t_us / passes_m / 1e3:.3f} ms of kernel time for {t_b / passes_m / 1e9:.2f} GB: "
                  f"{t_b / t_us / 1e3:.1f} GB/s ({t_b / t_us / 1e3 / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s)")
    pre = {}
    for r in rows:
        if re.search(r"gemm_tiles|splitk_reduce", r["Kernel_Name"]):
            k = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1))
            pre.setdefault(k, []).append(dur(r))
    if pre:
        print("prefill m = 512 kernels, per (kernel, grid):")
        print(f"{'kernel':44s} {'threads':>9s} {'n':>6s} {'avg us':>9s} {'median':>9s}")
        for (k, g), v in pre.items():
            print(f"{k[:44]:44s} {g:9d} {len(v):6d} {statistics.mean(v):9.2f} {statistics.median(v):9.2f}")


WAVE_STATE_COUNTERS = (("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
                        "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM"),
                       ("SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL",
                        "SQ_INST_LEVEL_LDS", "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_LDS",
                        "GRBM_GUI_ACTIVE"))


def summarize_wave_states(csv_a, csv_b, pattern="gemm_tiles|splitk_reduce|gemv|reconstruct"):
    """Where the waves of each library kernel spend their time, from two
    rocprofv3 --pmc runs of WAVE_STATE_COUNTERS (one per tuple): per (kernel,
    grid), the median per dispatch of each wave-state counter as a fraction
    of SQ_WAVE_CYCLES (waiting for a dependency or barrier, waiting to issue,
    issuing VALU / LDS / VMEM), MFMA busy over the SIMD cycles, and the LDS
    FIFO-full cycles over SQ_BUSY_CYCLES."""
    import csv
    import re

    def load(path):
        per = {}
        for r in csv.DictReader(open(path)):
            n = _short(r["Kernel_Name"])
            if not re.search(pattern, n):
                continue
            per.setdefault((n, int(r["Grid_Size"])), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        return {k: {c: statistics.median(v) for c, v in d.items()} for k, d in per.items()}

    a, b = load(csv_a), load(csv_b)
    print(f"{'kernel':46s} {'threads':>9s} {'wait dep':>8s} {'wait iss':>8s} {'wait LDS':>8s} {'issue':>6s} "
          f"{'VALU':>6s} {'LDS':>6s} {'VMEM':>6s} {'MFMA bz':>7s} {'LDS fifo':>8s}")
    for k, ca in a.items():
        cb = b.get(k, {})
        wc = ca.get("SQ_WAVE_CYCLES", 0.0)
        if not wc:
            continue
        f = lambda c: ca.get(c, 0.0) / wc
        simd = cb.get("GRBM_GUI_ACTIVE", 0.0) / 8 * 1024
        mb = cb.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / simd if simd else 0.0
        bz = cb.get("SQ_BUSY_CYCLES", 0.0)
        fifo = (cb.get("SQ_LDS_DATA_FIFO_FULL", 0.0) + cb.get("SQ_LDS_CMD_FIFO_FULL", 0.0)) / bz if bz else 0.0
        print(f"{k[0][:46]:46s} {k[1]:9d} {f('SQ_WAIT_ANY'):8.3f} {f('SQ_WAIT_INST_ANY'):8.3f} "
              f"{f('SQ_WAIT_INST_LDS'):8.3f} {f('SQ_ACTIVE_INST_ANY'):6.3f} {f('SQ_ACTIVE_INST_VALU'):6.3f} "
              f"{f('SQ_ACTIVE_INST_LDS'):6.3f} {f('SQ_ACTIVE_INST_VMEM'):6.3f} {mb:7.3f} {fifo:8.3f}")


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
                 "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU",
                 "GRBM_GUI_ACTIVE")


def summarize_mfma(counter_csv, gap=12):
    """MFMA use of the prefill / grouped kernels from a rocprofv3 --pmc run of
    MFMA_COUNTERS (its CSV carries each dispatch's start and end).  Per run of
    dispatches of one (kernel, grid): MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES
    over (GRBM_GUI_ACTIVE / 8 XCDs) x 1024 SIMDs, the average graphics clock =
    GRBM_GUI_ACTIVE / 8 over the dispatch's duration, and the MFMA rate
    (SQ_INSTS_MFMA x flop per instruction over the duration)."""
    import csv

    disp = {}
    for r in csv.DictReader(open(counter_csv)):
        name = _short(r["Kernel_Name"])
        if not ("gemm_tiles" in name or "splitk_reduce" in name or "ms_pass" in name or "ms_merge" in name):
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": name, "grid": int(r["Grid_Size"]),
                                                    "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3,
                                                    "c": {}})
        d["c"][r["Counter_Name"]] = float(r["Counter_Value"])
    runs, open_run = [], {}
    for i in sorted(disp):
        d = disp[i]
        k = (d["name"], d["grid"])
        # the MonoSoup kernels interleave with many small ones: one run per kernel
        if k in open_run and (i - open_run[k][0] <= gap or "ms_" in d["name"]):
            j = open_run[k][1]
        else:
            runs.append([k, i, []])
            j = len(runs) - 1
        runs[j][2].append(d)
        open_run[k] = (i, j)
    print(f"{'kernel':46s} {'threads':>9s} {'first':>6s} {'n':>3s} {'avg us':>8s} {'MFMA inst':>10s} "
          f"{'busy %':>6s} {'clock GHz':>9s} {'MFMA TF/s':>9s} {'VALU/MFMA':>9s} {'LDS/MFMA':>8s} {'bank cf':>7s}")
    for (name, threads), first, v in runs:
        us = statistics.mean(d["us"] for d in v)
        c = {n: statistics.mean(d["c"].get(n, 0.0) for d in v) for n in MFMA_COUNTERS}
        xcd_cycles = c["GRBM_GUI_ACTIVE"] / 8
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * 1024) if xcd_cycles else 0.0
        clock = xcd_cycles / us / 1e3 if us else 0.0
        mf = c["SQ_INSTS_MFMA"]
        # flop per MFMA instruction: v_mfma_f32_32x32x16_bf16 (prefill) or v_mfma_f32_32x32x2_f32 (MonoSoup)
        tf = mf * (4096 if "ms_" in name else 32768) / us / 1e6 if us else 0.0
        per = (f"{c['SQ_INSTS_VALU'] / mf:9.2f} {c['SQ_INSTS_LDS'] / mf:8.2f}" if mf else f"{'-':>9s} {'-':>8s}")
        print(f"{name[:46]:46s} {threads:9d} {first:6d} {len(v):3d} {us:8.1f} {mf:10.0f} "
              f"{100 * busy:6.1f} {clock:9.2f} {tf:9.0f} {per} {c['SQ_LDS_BANK_CONFLICT']:7.0f}")


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.copy_mb, args.command)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_stack:
        summarize_stack(args.summarize_stack, args.stack_layers)
        return
    if args.summarize_wave_states:
        summarize_wave_states(*args.summarize_wave_states)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_kernels:
        summarize_kernels(*args.summarize_kernels)
        return
    if args.summarize_gemm_counters:
        e, f, w, mb = args.summarize_gemm_counters
        summarize_gemm_counters(e, f, w, int(mb), args.command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              f"Sharding is described in the design notes; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    import synth
    import tenant_fine_tune_amd as bd

    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.stack:
        res = run_stack(torch, bd, synth, args.stack_layers)
        line = {"metric": METRIC, "value": res["decode"]["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": 10,
                "warmup": 1, "ms_per_step": res["decode"]["ms"], "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                "config": {"workload": f"70B-shaped linear stack, {args.stack_layers} layers x 7 linears, 14 packed "
                                       f"delta sets resident; value = 1-token decode pass through every linear",
                           "parallelism": "single GPU"},
                "stack": res}
        print(json.dumps(line), flush=True)
        return
    if args.no_decode:
        value = ms_per_step = roofline = step_bytes = None
        kernels, rooflines = {}, {}
    else:
        ds, dev_s, wall_s, kernels = run_decode(torch, bd, synth, args.steps, args.warmup, args.kernel_reps)
        ms_per_step = dev_s / args.steps * 1e3
        value = ds.step_bytes * args.steps / dev_s / 1e9
        log(f"decode step (fused linear m=1,4,16 x 2 alpha modes): {ms_per_step * 1e3:.2f} us/step, "
            f"{value:.1f} GB/s (wall {wall_s * 1e3:.1f} ms for {args.steps} steps)")
        for k, v in kernels.items():
            log(f"  {k:22s} {v['us']:8.2f} us  {v['GB/s']:8.1f} GB/s  {100 * v['frac_hbm']:.1f}% of HBM")
        rooflines = {k: hbm_roofline(k, kernels[k]) for k in STEP + OFFLINE}
        # dominant kernel: the step entry with the largest launch time
        dom = max(STEP, key=lambda k: kernels[k]["us"])
        roofline = rooflines[dom]
        step_bytes = ds.step_bytes
        del ds
        torch.cuda.empty_cache()

    prefill = None if args.no_prefill else run_prefill(torch, bd, synth, only=args.prefill_shapes)
    if prefill is not None:
        for label, e in prefill["shapes"].items():
            rooflines[f"prefill_{label}"] = e["roofline"]
    grouped, similarity = (None, None) if args.no_grouped else run_grouped(torch, bd, synth, rows=args.grouped_rows)
    if grouped is not None:
        rooflines["grouped"] = grouped["roofline"]
    monosoup = None if args.no_monosoup else run_monosoup(torch, bd, synth)
    context = None if args.no_context else run_context(torch, only=args.prefill_shapes)
    if context is not None:
        context["probes"] = pr = run_probes(torch, bd)
        # each roofline against what the chip sustains as well: HBM-bound
        # entries over the read probe on the same 34 MiB rotation (up to
        # 64 MiB per launch: the decode linears) or on 1 GiB (compress,
        # reconstruct), MFMA-bound ones over the MFMA probe
        for k, r in rooflines.items():
            if r["bound"] == "hbm":
                ref = pr["read_34MiB" if r["algorithmic_bytes_per_launch"] <= (64 << 20) else "read_1GiB"]
                r["frac_of_read_probe"] = round(r["achieved"] / ref["GB/s"], 4)
            else:
                r["frac_of_mfma_probe"] = round(r["achieved"] / pr["mfma_bf16"]["TFLOP/s"], 4)
    if context is not None and prefill is not None:
        context["unfused_m2048"] = run_unfused(torch, bd, synth, prefill, only=args.prefill_shapes)
    torch.cuda.empty_cache()
    stack = None if args.no_stack else run_stack(torch, bd, synth, args.stack_layers)
    torch.cuda.empty_cache()
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(args.cpu_seconds)
    if not args.no_cpu_baseline:
        if prefill is not None:
            prefill["cpu_oracle"] = run_cpu_prefill()
        if grouped is not None:
            grouped["cpu_oracle"] = run_cpu_grouped(grouped["group_sizes"])
        if stack is not None:
            stack["cpu_oracle"] = run_cpu_stack(args.stack_layers)

    line = {
        "metric": METRIC,
        "value": round(value, 1) if value is not None else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5) if ms_per_step is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode layer 4096x4096 bf16 + packed 1-bit deltas through the fused linear: "
                               "m=1,4,16 tokens with row and matrix alpha; 16 rotating weight sets",
                   "d_out": R, "d_in": C, "m": list(DECODE_M), "weight_sets": SETS, "parallelism": "single GPU",
                   "step_bytes": step_bytes},
        "roofline": roofline,
        "rooflines": rooflines,
        "kernels": kernels,
        "prefill": prefill,
        "grouped": grouped,
        "similarity": similarity,
        "monosoup": monosoup,
        "stack": stack,
        "context": context,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read + {n} bytes written")


if __name__ == "__main__":
    main()

"""Benchmark of the quantized MoE FFN layer on one MI355X.

The headline line is decode: one call of the whole layer (router, top-k,
routed experts, shared expert, combine) for one token of a Gemma-4-26B-A4B-
shaped layer (hidden 2816, 128 experts, top-8, expert intermediate 704,
shared intermediate 2112; 8-bit router, 4-bit experts, group 64).  Calls
rotate over --layers distinct resident layers with a fresh token each, so
the 256 MB Infinity Cache cannot hold the working set, and every timed
replay follows an untimed 1 GiB streaming read that evicts it.  The timed
calls are replayed from a HIP graph (one capture of K calls); the figure is
the median over five replays, and the workspace's error bits are checked
after every timed region.  Inputs are resident in HBM before the timer
starts.  The HBM read peak is also measured (mq_stream_read over 4 GiB) and
fractions are given against both it and the vendor figure.  The single-launch decode kernel's own duration
is the timed region's event interval over the launches in it (one launch
per call); the roofline figure divides the call's algorithmic bytes by it.

Also reported (extra fields of the same JSON line): the 128-token prefill
chunk with Zipf(1.1)-skewed routing, the 30-layer stack (one token through
30 layers, each call normalising its input), the 4096-token prefill (the
matrix-core regime, reported in TFLOP/s), and the fp64 CPU oracle timed on
bounded samples of decode and prefill tokens, on one core and on all host
cores.  Prints one JSON line on stdout.

Profiling helpers (not part of the default run):
  --profile decode       runs decode calls back to back, then a copy kernel of
                         known size, for rocprofv3 counter runs;
  --profile prefill      runs 128-token prefill calls (Zipf-skewed routing)
                         back to back, for counter runs on the grouped kernels;
  --profile large        runs 4096-token prefill calls (Zipf-skewed routing)
                         back to back, for matrix-core counter runs;
  --traffic-summary F W  turns the FETCH_SIZE / WRITE_SIZE counter CSVs of
                         those runs into the traffic summary under profiles/;
  --prefill-summary F W S  turns FETCH_SIZE / WRITE_SIZE counter CSVs and the
                         kernel statistics CSV of --profile prefill runs into
                         the per-kernel traffic summary of the grouped path;
  --counters-summary A B S  turns the two SQ counter passes (COUNTERS_A,
                         COUNTERS_B) and the kernel statistics of --profile
                         large runs into the matrix-core/LDS utilisation
                         table under profiles/;
  --stats-summary S J    turns the kernel statistics CSV of a rocprofv3
                         --kernel-trace --stats run of the default benchmark,
                         and the JSON line that run printed, into the kernel
                         table under profiles/.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 matrix peak, vendor figure
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (% of peak), decode and 128-tok prefill"
DECODE_KERNEL = "k_decode"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_decode_decode_h2816_e128_traffic.txt")
STATS_FILE = os.path.join(ROOT, "profiles", "kernel_stats_bench_decode_prefill128_stack30_prefill4096.txt")
PREFILL_FILE = os.path.join(ROOT, "profiles", "grouped_kernels_prefill128_h2816_e128_traffic.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "grouped_kernels_prefill4096_h2816_e128_counters.txt")
# The copy kernel's FETCH_SIZE reads half its bytes (see the decode traffic summary).
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
COPY_BYTES = 256 << 20       # each direction of the reference copy kernel
# Sources whose change invalidates the recorded counter traffic of the decode kernel.
KERNEL_SOURCES = ["fused.hip", "decode_units.h", "device.h", "plan.h", "layout.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_moe_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def build_layers(M, S, cfg, seed, n_layers, threads):
    """n_layers distinct layers resident on the GPU (generated and packed per expert in parallel)."""
    layers = []
    pool = M.pool_layout(cfg.hidden, cfg.inter)
    for l in range(n_layers):
        t0 = time.time()
        src = S.make_layer(cfg, seed, layer=l, experts=False)
        host = np.zeros(cfg.num_experts * pool.expert_stride, dtype=np.uint8)

        def one(e):
            g, u, d = S.make_expert(cfg, seed, l, e)
            M.pack_expert_into(pool, e, g, u, d, host)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(cfg.num_experts)))
        layers.append(M.DeviceLayer(src, pool_host=host))
        del host
        log("layer %d resident (%.1f s)" % (l, time.time() - t0))
    return layers


def layer_bytes(M, cfg):
    """Algorithmic bytes: one routed expert, the router, the shared expert."""
    H, I, Is = cfg.hidden, cfg.inter, cfg.shared_inter
    expert = 2 * M.packed_bytes(I, H, 4) + M.packed_bytes(H, I, 4)
    shared = 2 * M.packed_bytes(Is, H, 4) + M.packed_bytes(H, Is, 4)
    router = M.packed_bytes(cfg.num_experts, H, 8)
    return expert, router, shared


def flops_per_token(cfg):
    H, E, k, I, Is = cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter, cfg.shared_inter
    return 2 * E * H + k * 6 * I * H + 6 * Is * H


def time_graph(torch, calls, steps, warmup, flush=None, reps=5):
    """Capture `steps` calls in one HIP graph; warm up, then time `reps`
    replays, each preceded by the untimed `flush` (a streaming read that
    evicts the Infinity Cache).  Returns the median ms per call, the per-replay
    values and the graph."""
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                calls[i % len(calls)]()
    torch.cuda.synchronize()
    g.replay()                      # untimed replay
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        if flush is not None:
            flush()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        per.append(ev0.elapsed_time(ev1) / steps)
    return float(np.median(per)), per, g


class Flush:
    """Streaming reads over a buffer larger than the Infinity Cache: run
    before each timed replay so that no weights of the timed calls are cached
    from earlier work, and timed on its own as the measured HBM read peak."""

    def __init__(self, torch, M, nbytes=4 << 30, workgroups=4096):
        self.torch, self.M, self.wg = torch, M, workgroups
        self.buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        self.small = self.buf[: (1 << 30) // 4]
        self.sink = torch.empty(workgroups, dtype=torch.int32, device="cuda")

    def __call__(self):
        self.M.stream_read(self.small, self.sink, self.wg)

    def peak_gbs(self, reps=5):
        torch = self.torch
        for _ in range(2):
            self.M.stream_read(self.buf, self.sink, self.wg)
        per = []
        for _ in range(reps):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            self.M.stream_read(self.buf, self.sink, self.wg)
            ev1.record()
            torch.cuda.synchronize()
            per.append(self.buf.numel() * 4 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9)
        return float(np.median(per)), per


def time_eager(torch, calls, steps):
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        calls[i % len(calls)]()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def recorded_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None
    when it is missing or was taken from other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            txt = f.read()
    except OSError:
        return None, "no counter summary"
    kv = dict(re.findall(r"^(\w+):\s*(\S+)\s*$", txt, re.M))
    if kv.get("source_sha256") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return float(kv["traffic_bytes_per_launch"]), "rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(S, cfg, seed, threads, reps=5):
    """The fp64 C oracle on the host cores: decode tokens of one layer of the
    decode workload and 128-token prefill rows of the same layer with the
    Zipf skew, on one core and on `threads` cores (tokens split over
    threads), median of `reps` runs each, input generation excluded."""
    import oracle as O
    host = S.make_layer(cfg, seed, layer=0)
    zhost = S.make_layer(cfg, seed, layer=0)
    zhost.logit_bias = S.zipf_logit_bias(seed, 0, cfg.num_experts)

    def rate(layer, x, n_thr):
        per = []
        for _ in range(reps):
            t0 = time.time()
            O.forward(layer, x, threads=n_thr, dense_experts=False)
            per.append(x.shape[0] / (time.time() - t0))
        return float(np.median(per))
    xd = S.make_tokens(seed, threads, cfg.hidden, batch=7)
    xp = S.make_tokens(seed, 128, cfg.hidden, batch=8)
    t0 = time.time()
    res = {
        "decode_1core": rate(host, xd[:1], 1),
        "decode_all_cores": rate(host, xd, threads),
        "prefill128_1core": rate(zhost, xp[:4], 1),
        "prefill128_all_cores": rate(zhost, xp, threads),
    }
    wall = time.time() - t0
    return dict(value=res["decode_all_cores"], unit="tokens/s", cores=threads, kind="oracle",
                sample="decode: %d tokens of one layer of the decode workload, one per thread on %d threads "
                       "(1 token on 1 core); prefill128: the 128 rows of one chunk with the Zipf skew on %d "
                       "threads (4 of them on 1 core); fp64 C oracle, median of %d runs each, %.0f s wall in all"
                       % (threads, threads, threads, reps, wall),
                host_cpu=cpu_model(), host_nproc=os.cpu_count(),
                **{k + "_tokens_per_s": v for k, v in res.items()})


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


# ------------------------------------------------------------------ profiling helpers

def profile_decode(args):
    """Back-to-back decode calls, then a copy kernel of COPY_BYTES each way."""
    import torch
    import qmoe_synth as S
    import quantized_moe_gemv_amd as M
    torch.cuda.set_device(0)
    cfg, seed = S.CONFIGS["decode"], S.SEEDS["stack30"]
    layers = build_layers(M, S, cfg, seed, args.layers, host_threads())
    xs = torch.from_numpy(S.make_tokens(seed, args.steps, cfg.hidden, batch=1).view(np.int16)).view(torch.bfloat16)
    xs = xs.cuda()
    ws = layers[0].new_workspace(1)
    out = torch.empty((1, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    for i in range(args.steps):
        M.moe_layer_forward(layers[i % len(layers)], xs[i:i + 1], out=out, workspace=ws, path="fused")
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log("profile run done: %d decode calls, 5 copies of %d B" % (args.steps, COPY_BYTES))


def profile_prefill(args):
    """Back-to-back 128-token prefill calls over the resident layers."""
    import torch
    import qmoe_synth as S
    import quantized_moe_gemv_amd as M
    torch.cuda.set_device(0)
    cfg, seed, T = S.CONFIGS["decode"], S.SEEDS["stack30"], 128
    layers = build_layers(M, S, cfg, seed, args.layers, host_threads())
    zl = [d.with_logit_bias(torch.from_numpy(S.zipf_logit_bias(seed, l, cfg.num_experts)).cuda())
          for l, d in enumerate(layers)]
    nb = max(1, min(args.steps, 2 * len(layers)))
    xp = torch.from_numpy(S.make_tokens(seed, nb * T, cfg.hidden, batch=2).view(np.int16)).view(torch.bfloat16)
    xp = xp.cuda().view(nb, T, cfg.hidden)
    ws = layers[0].new_workspace(T)
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    for i in range(args.steps):
        M.moe_layer_forward(zl[i % len(zl)], xp[i % nb], out=out, workspace=ws)
    torch.cuda.synchronize()
    log("profile run done: %d prefill calls of %d tokens" % (args.steps, T))


def profile_large(args):
    """Back-to-back 4096-token prefill calls on one layer."""
    import torch
    import qmoe_synth as S
    import quantized_moe_gemv_amd as M
    torch.cuda.set_device(0)
    cfg, seed, T = S.CONFIGS["decode"], S.SEEDS["stack30"], 4096
    layers = build_layers(M, S, cfg, seed, 1, host_threads())
    dev = layers[0].with_logit_bias(torch.from_numpy(S.zipf_logit_bias(seed, 0, cfg.num_experts)).cuda())
    xl = torch.from_numpy(S.make_tokens(seed, T, cfg.hidden, batch=4).view(np.int16)).view(torch.bfloat16).cuda()
    ws = dev.new_workspace(T)
    out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    for i in range(args.steps):
        M.moe_layer_forward(dev, xl, out=out, workspace=ws)
        torch.cuda.synchronize()
        log("large call %d done" % i)
    errs = M.workspace_errors(ws)
    if errs:
        raise SystemExit("prefill4096: workspace error bits 0x%x" % errs)
    log("profile run done: %d prefill calls of %d tokens" % (args.steps, T))


def read_counter(path, counter):
    """Per-dispatch values of `counter` for the decode kernel and the copy kernel."""
    dec, cop = [], []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if DECODE_KERNEL in r["Kernel_Name"]:
                dec.append(v)
            elif "elementwise_kernel" in r["Kernel_Name"] and int(r["Grid_Size"]) >= COPY_BYTES // 64:
                cop.append(v)
    if not dec or not cop:
        raise SystemExit("%s: no %s rows for the decode or the copy kernel" % (path, counter))
    return float(np.median(dec)), float(np.median(cop)), len(dec)


def traffic_summary(fetch_csv, write_csv, out_path):
    f_dec, f_cop, n = read_counter(fetch_csv, "FETCH_SIZE")
    w_dec, w_cop, _ = read_counter(write_csv, "WRITE_SIZE")
    ff = COPY_BYTES / (f_cop * 1024.0)     # bytes per KiB of counter reading
    fw = COPY_BYTES / (w_cop * 1024.0)
    fetch = f_dec * 1024.0 * ff
    write = w_dec * 1024.0 * fw
    lines = [
        "# HBM traffic of the single-launch decode kernel (k_decode)",
        "# workload: decode, 1 token per call, H2816 E128 top8 I704 Is2112, rotated over 30 resident layers",
        "# commands (run from /tmp with TMPDIR=/tmp):",
        "#   rocprofv3 --pmc FETCH_SIZE -d <dir> -o fetch --output-format csv -- python3 <repo>/bench.py --profile decode --steps 200",
        "#   rocprofv3 --pmc WRITE_SIZE -d <dir> -o write --output-format csv -- python3 <repo>/bench.py --profile decode --steps 200",
        "#   python3 <repo>/bench.py --traffic-summary <dir>/fetch_counter_collection.csv <dir>/write_counter_collection.csv",
        "# The copy kernel (torch.neg over %d B, fp32) reads and writes %d B per launch; its counter" % (COPY_BYTES, COPY_BYTES),
        "# readings give the scale from KiB of counter to bytes of HBM traffic.",
        "kernel: %s" % DECODE_KERNEL,
        "source_sha256: %s" % kernel_source_hash(),
        "dispatches: %d" % n,
        "fetch_kib_per_dispatch: %.1f" % f_dec,
        "write_kib_per_dispatch: %.1f" % w_dec,
        "copy_fetch_kib: %.1f" % f_cop,
        "copy_write_kib: %.1f" % w_cop,
        "fetch_scale: %.4f" % ff,
        "write_scale: %.4f" % fw,
        "fetch_bytes_per_launch: %.0f" % fetch,
        "write_bytes_per_launch: %.0f" % write,
        "traffic_bytes_per_launch: %.0f" % (fetch + write),
        "algorithmic_bytes_per_launch: 37193728",
    ]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def prefill_summary(fetch_csv, write_csv, stats_csv, out_path):
    """Per grouped-path kernel: HBM bytes per dispatch (counters scaled as for
    the decode kernel) and the average duration, for 128-token prefill calls."""
    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: float(np.median(v)) for k, v in vals.items()}
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    with open(stats_csv) as f:
        dur = {r["Name"]: float(r["AverageNs"]) / 1e3 for r in csv.DictReader(f)}
    lines = [
        "# HBM traffic and duration per kernel of the grouped path, 128-token prefill",
        "# workload: 128 tokens per call, Zipf(1.1) logit bias, H2816 E128 top8 I704 Is2112, rotated over 6 layers",
        "# commands (run from /tmp with TMPDIR=/tmp):",
        "#   rocprofv3 --pmc FETCH_SIZE -d <dir> -o pfetch --output-format csv -- python3 <repo>/bench.py --profile prefill --steps 60 --layers 6",
        "#   rocprofv3 --pmc WRITE_SIZE -d <dir> -o pwrite --output-format csv -- python3 <repo>/bench.py --profile prefill --steps 60 --layers 6",
        "#   rocprofv3 --kernel-trace --stats -d <dir> -o pstats --output-format csv -- python3 <repo>/bench.py --profile prefill --steps 60 --layers 6",
        "#   python3 <repo>/bench.py --prefill-summary <fetch csv> <write csv> <pstats_kernel_stats.csv>",
        "# counter KiB scaled by %.1f (FETCH_SIZE) and %.1f (WRITE_SIZE), as in the decode traffic summary" % (FETCH_SCALE, WRITE_SCALE),
        "# (the FETCH_SIZE scale was measured on 128-byte line requests; a kernel whose requests are",
        "# partly 64-byte, as the down projection's 8-byte-per-lane loads may be, reads less than shown)",
        "",
        "%-34s %10s %10s %10s %10s" % ("kernel", "read_MB", "write_MB", "avg_us", "GB/s"),
    ]
    for name in sorted(fetch, key=lambda n: -fetch[n]):
        short = name.split("(")[0].replace("void ", "")
        rd = fetch[name] * 1024 * FETCH_SCALE / 1e6
        wr = write.get(name, 0.0) * 1024 * WRITE_SCALE / 1e6
        us = next((v for k, v in dur.items() if k.startswith(name.split("(")[0])), float("nan"))
        lines.append("%-34s %10.1f %10.1f %10.2f %10.0f" % (short, rd, wr, us, (rd + wr) * 1e3 / us))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


COUNTERS_A = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_LDS_IDX_ACTIVE "
              "SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE")
COUNTERS_B = ("SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS "
              "SQ_ACTIVE_INST_VMEM SQ_WAVES GRBM_GUI_ACTIVE")


def counters_summary(a_csv, b_csv, stats_csv, out_path):
    """Matrix-core, VALU and LDS utilisation per grouped-path kernel of the
    4096-token prefill, from two SQ counter passes (the rocprof derived
    metrics' formulas, written out)."""
    vals = {}
    for path in (a_csv, b_csv):
        with open(path) as f:
            for r in csv.DictReader(f):
                vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    with open(stats_csv) as f:
        dur = {r["Name"]: float(r["AverageNs"]) / 1e3 for r in csv.DictReader(f)}
    simds, cus, xcds = 1024, 256, 8
    lines = [
        "# Matrix-core, VALU and LDS utilisation per kernel of the grouped path, 4096-token prefill",
        "# workload: 4096 tokens, Zipf(1.1) logit bias, H2816 E128 top8 I704 Is2112, one layer",
        "# commands (run from /tmp with TMPDIR=/tmp; each counter pass in a run of its own):",
        "#   rocprofv3 --kernel-trace --stats -d <dir> -o st --output-format csv -- python3 <repo>/bench.py --profile large --steps 4",
        "#   rocprofv3 --pmc %s -d <dir> -o pa --output-format csv -- python3 <repo>/bench.py --profile large --steps 2" % COUNTERS_A,
        "#   rocprofv3 --pmc %s -d <dir> -o pb --output-format csv -- python3 <repo>/bench.py --profile large --steps 2" % COUNTERS_B,
        "#   python3 <repo>/bench.py --counters-summary <pa csv> <pb csv> <st_kernel_stats.csv>",
        "# GRBM_GUI_ACTIVE comes summed over the %d XCDs; one XCD's busy cycles G = value / %d." % (xcds, xcds),
        "# mfma% = SQ_VALU_MFMA_BUSY_CYCLES / (G * 1024 SIMDs) (a 16x16x32 fp16 MFMA counts 16 cycles: the",
        "#   2.5 PFLOP/s peak at 2.4 GHz); valu% = SQ_ACTIVE_INST_VALU / (G * 256 CUs); lds% = SQ_LDS_IDX_ACTIVE /",
        "#   (G * 256); conflict% = SQ_LDS_BANK_CONFLICT / (G * 256); wait% = SQ_WAIT_ANY / SQ_WAVE_CYCLES (wave",
        "#   time waiting on a counter: memory, LDS or a barrier); issue% = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.",
        "",
        "%-22s %8s %6s %6s %6s %9s %6s %6s %9s %9s %8s" % ("kernel", "avg_us", "mfma%", "valu%", "lds%", "conflict%",
                                                          "wait%", "issue%", "mfma_M", "valu_M", "lds_M"),
    ]
    for name in sorted(vals, key=lambda n: -dur.get(n, next((v for k, v in dur.items() if k.startswith(n.split("(")[0])), 0))):
        if "mq::" not in name:
            continue
        v = {c: float(np.median(x)) for c, x in vals[name].items()}
        g = v["GRBM_GUI_ACTIVE"] / xcds
        us = next((d for k, d in dur.items() if k.startswith(name.split("(")[0])), float("nan"))
        lines.append("%-22s %8.1f %6.1f %6.1f %6.1f %9.1f %6.1f %6.1f %9.2f %9.2f %8.2f" % (
            name.split("(")[0].replace("void ", "").replace("mq::", ""), us,
            100 * v["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * simds), 100 * v["SQ_ACTIVE_INST_VALU"] / (g * cus),
            100 * v["SQ_LDS_IDX_ACTIVE"] / (g * cus), 100 * v["SQ_LDS_BANK_CONFLICT"] / (g * cus),
            100 * v["SQ_WAIT_ANY"] / v["SQ_WAVE_CYCLES"], 100 * v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"],
            v["SQ_INSTS_MFMA"] / 1e6, v["SQ_INSTS_VALU"] / 1e6, v["SQ_INSTS_LDS"] / 1e6))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_summary(stats_csv, bench_json, out_path):
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    with open(bench_json) as f:
        res = json.loads([l for l in f if l.strip().startswith("{")][-1])
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [
        "# rocprofv3 kernel statistics of the default benchmark run",
        "# workloads: decode (graph of %d calls + eager calls, %d resident layers), 128-token prefill (graph),"
        % (res["steps"], res["config"].get("resident_layers", 30)),
        "#            30-layer stack with RMSNorm, 4096-token prefill (graph); warm-up calls included",
        "# command (from /tmp with TMPDIR=/tmp):",
        "#   rocprofv3 --kernel-trace --stats -d <dir> -o bench --output-format csv -- python3 <repo>/bench.py > <dir>/bench.json",
        "#   python3 <repo>/bench.py --stats-summary <dir>/bench_kernel_stats.csv <dir>/bench.json",
        "# bench.py in the same run: decode %.2f us/call (graph)" % (res["ms_per_step"] * 1000.0),
    ]
    extra = []
    if isinstance(res.get("prefill128"), dict):
        extra.append("prefill128 %.2f us/call" % (res["prefill128"]["ms_per_call"] * 1e3))
    if isinstance(res.get("stack"), dict):
        extra.append("stack%d %.2f us/token" % (res["stack"]["layers"], res["stack"]["ms_per_token"] * 1e3))
    if isinstance(res.get("prefill4096"), dict):
        extra.append("prefill4096 %.3f ms/call" % res["prefill4096"]["ms_per_call"])
    if extra:
        lines.append("#   " + ", ".join(extra))
    lines += ["", "%-62s %6s %12s %10s %10s %10s" % ("kernel", "calls", "total_ms", "avg_us", "min_us", "max_us")]
    for r in rows:
        name = r["Name"]
        name = name if len(name) <= 60 else name[:57] + "..."
        lines.append("%-62s %6d %12.3f %10.2f %10.2f %10.2f" % (
            name, int(r["Calls"]), float(r["TotalDurationNs"]) / 1e6, float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------------ main run

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--prefill-steps", type=int, default=60)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-large", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "gemv", "grouped"])
    ap.add_argument("--profile", choices=["decode", "prefill", "large"])
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "BENCH_JSON"))
    ap.add_argument("--prefill-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "STATS_CSV"))
    ap.add_argument("--counters-summary", nargs=3, metavar=("PASS_A_CSV", "PASS_B_CSV", "STATS_CSV"))
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1], TRAFFIC_FILE)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary[0], args.stats_summary[1], STATS_FILE)
        return
    if args.prefill_summary:
        prefill_summary(*args.prefill_summary, PREFILL_FILE)
        return
    if args.counters_summary:
        counters_summary(*args.counters_summary, COUNTERS_FILE)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X and has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.profile == "decode":
        profile_decode(args)
        return
    if args.profile == "prefill":
        profile_prefill(args)
        return
    if args.profile == "large":
        profile_large(args)
        return

    import torch
    import qmoe_synth as S
    import quantized_moe_gemv_amd as M

    torch.cuda.set_device(0)
    cfg = S.CONFIGS["decode"]
    seed = S.SEEDS["stack30"]
    threads = host_threads()
    layers = build_layers(M, S, cfg, seed, args.layers, threads)
    H, k = cfg.hidden, cfg.top_k
    expert_b, router_b, shared_b = layer_bytes(M, cfg)
    per_call = router_b + k * expert_b + shared_b + 2 * H * 2

    flush = Flush(torch, M)
    peak, peak_all = flush.peak_gbs()
    log("streaming read of %.1f GiB: %.0f GB/s (median of %d)" % (flush.buf.numel() * 4 / 2 ** 30, peak, len(peak_all)))

    def errors_clear(ws_, what):
        bits = M.workspace_errors(ws_)
        if bits != 0:
            raise SystemExit("%s: workspace error bits 0x%x after the timed calls" % (what, bits))

    # ---------------------------------------------------------------- decode
    n_tok = args.steps
    xs = S.make_tokens(seed, n_tok, H, batch=1)
    xdev = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).cuda()
    ws = layers[0].new_workspace(128)
    out = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")

    def decode_call(i):
        dev = layers[i % len(layers)]
        x = xdev[i % n_tok:i % n_tok + 1]
        return lambda: M.moe_layer_forward(dev, x, out=out, workspace=ws, path=args.path)
    calls = [decode_call(i) for i in range(args.steps)]
    ms, ms_all, _ = time_graph(torch, calls, args.steps, args.warmup, flush)
    errors_clear(ws, "decode")
    ms_eager = time_eager(torch, calls, min(args.steps, 300))
    errors_clear(ws, "decode (eager)")
    # one launch of the decode kernel per call: the timed region's events over its launches
    gbs = per_call / (ms * 1e-3) / 1e9
    log("decode: %.2f us/call (graph), %.2f us/call (eager), %.0f GB/s" % (ms * 1e3, ms_eager * 1e3, gbs))
    traffic, traffic_note = recorded_traffic() if args.path in ("auto", "fused") else (None, "not the fused kernel")

    result = {
        "metric": METRIC,
        "value": 1.0 / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded uniform 4-bit/8-bit group-64 affine codes, bf16 scale/bias, bf16 N(0,1) tokens)",
        "config": {
            "workload": "decode, 1 token per call, Gemma-4-26B-A4B-shaped MoE layer (hidden 2816, 128 experts, "
                        "top-8, expert intermediate 704, shared intermediate 2112; 8-bit router, 4-bit experts, "
                        "group 64), rotated over %d resident layers" % len(layers),
            "tokens_per_call": 1, "resident_layers": len(layers),
            "distinct_layers_per_replay": min(args.steps, len(layers)),
            "launch": "hip graph of %d calls; median of %d replays, each after a 1 GiB streaming read that "
                      "evicts the Infinity Cache" % (args.steps, len(ms_all)),
            "weights": "int4/int8 affine group-64, bf16 scale+bias", "accumulate": "fp32", "output": "bf16",
            "path": args.path,
        },
        "roofline": {
            "bound": "hbm", "kernel": DECODE_KERNEL if args.path in ("auto", "fused") else "whole call",
            "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic, "traffic_source": traffic_note,
            "algorithmic_bytes_per_launch": per_call, "launch_ms": ms,
            "launch_ms_per_replay": ms_all,
            "measured_peak": peak, "frac_measured_peak": gbs / peak,
            "measured_peak_source": "mq_stream_read over 4 GiB, 16-byte streaming loads, median of 5",
        },
        "decode_eager_ms_per_call": ms_eager,
    }

    # ---------------------------------------------------------------- prefill 128
    if not args.no_prefill:
        T = 128
        nb = max(1, min(args.prefill_steps, 2 * len(layers)))
        xp = torch.from_numpy(S.make_tokens(seed, nb * T, H, batch=2).view(np.int16)).view(torch.bfloat16).cuda()
        xp = xp.view(nb, T, H)
        biases = [torch.from_numpy(S.zipf_logit_bias(seed, l, cfg.num_experts)).cuda() for l in range(len(layers))]
        zl = [d.with_logit_bias(b) for d, b in zip(layers, biases)]
        outp = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((nb, T, k), dtype=torch.int32, device="cuda")

        def prefill_call(i):
            dev = zl[i % len(zl)]
            return lambda: M.moe_layer_forward(dev, xp[i % nb], out=outp, workspace=ws, topk_ids=ids[i % nb])
        pcalls = [prefill_call(i) for i in range(args.prefill_steps)]
        pms, pms_all, _ = time_graph(torch, pcalls, args.prefill_steps, max(2, args.warmup // 10), flush)
        errors_clear(ws, "prefill128")
        idh = ids.cpu().numpy()
        touched = np.array([len(np.unique(idh[i % nb])) for i in range(args.prefill_steps)])
        pbytes = router_b + touched.mean() * expert_b + shared_b + 2 * T * H * 2
        pgbs = pbytes / (pms * 1e-3) / 1e9
        log("prefill128: %.2f us/call, %.0f tokens/s, %.0f GB/s, %.1f experts touched" %
            (pms * 1e3, T / (pms * 1e-3), pgbs, touched.mean()))
        result["prefill128"] = {
            "tokens_per_s": T / (pms * 1e-3), "ms_per_call": pms, "achieved_GBs": pgbs,
            "frac_hbm_peak": pgbs / HBM_PEAK_GBS, "frac_measured_peak": pgbs / peak,
            "ms_per_call_per_replay": pms_all, "experts_touched_mean": float(touched.mean()),
            "bytes_per_call": float(pbytes), "calls": args.prefill_steps,
            "workload": "128-token prefill chunk, Zipf(1.1) logit bias, same layers",
        }

    # ---------------------------------------------------------------- 30-layer stack
    if not args.no_stack and len(layers) >= 2:
        ntk = 8
        xa = torch.from_numpy(S.make_tokens(seed, ntk, H, batch=3).view(np.int16)).view(torch.bfloat16).cuda()
        # one launch per token through every layer (moe_stack_forward)
        stack = M.Stack(layers)
        sws = stack.new_workspace()
        sout = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
        scalls = [lambda t=t: M.moe_stack_forward(stack, xa[t:t + 1], out=sout, workspace=sws, between_eps=cfg.eps)
                  for t in range(ntk)]
        per_tok, _, _ = time_graph(torch, scalls, len(scalls), 2, flush)
        errors_clear(sws, "stack")
        # the same stack as one single-launch call per layer
        bufs = [torch.empty((1, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]

        def token_calls(t):
            seq = []
            for l, dev in enumerate(layers):
                src = xa[t:t + 1] if l == 0 else bufs[l % 2]
                dst = bufs[(l + 1) % 2]
                # layers after the first normalise their input inside the call
                e = 0.0 if l == 0 else cfg.eps
                seq.append(lambda dev=dev, src=src, dst=dst, e=e:
                           M.moe_layer_forward(dev, src, out=dst, workspace=ws, input_rmsnorm_eps=e))
            return seq
        lcalls = [c for t in range(ntk) for c in token_calls(t)]
        lms, _, _ = time_graph(torch, lcalls, len(lcalls), 0, flush)
        errors_clear(ws, "stack as layer calls")
        per_tok_calls = lms * len(lcalls) / ntk
        sgbs = len(layers) * per_call / (per_tok * 1e-3) / 1e9
        log("stack%d: %.2f us/token, %.0f tokens/s, %.0f GB/s (one launch per token); %.2f us/token as %d layer calls"
            % (len(layers), per_tok * 1e3, 1.0 / (per_tok * 1e-3), sgbs, per_tok_calls * 1e3, len(layers)))
        result["stack"] = {
            "layers": len(layers), "tokens_per_s": 1.0 / (per_tok * 1e-3), "ms_per_token": per_tok,
            "achieved_GBs": sgbs, "frac_hbm_peak": sgbs / HBM_PEAK_GBS, "frac_measured_peak": sgbs / peak,
            "tokens": ntk,
            "launch": "moe_stack_forward: one launch per token through every layer (hip graph of %d tokens)" % ntk,
            "layer_calls_ms_per_token": per_tok_calls,
            "workload": "one decode token through %d resident layers, unit-weight RMSNorm between layers" % len(layers),
        }

    # ---------------------------------------------------------------- prefill 4096
    if not args.no_large:
        T = 4096
        xl = torch.from_numpy(S.make_tokens(seed, T, H, batch=4).view(np.int16)).view(torch.bfloat16).cuda()
        zb = torch.from_numpy(S.zipf_logit_bias(seed, 0, cfg.num_experts)).cuda()
        dev = layers[0].with_logit_bias(zb)
        wsl = dev.new_workspace(T)
        outl = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        lcall = [lambda: M.moe_layer_forward(dev, xl, out=outl, workspace=wsl)]
        lms, _, _ = time_graph(torch, lcall, 3, 1, flush)
        errors_clear(wsl, "prefill4096")
        tf = T * flops_per_token(cfg) / (lms * 1e-3) / 1e12
        log("prefill4096: %.3f ms/call, %.0f tokens/s, %.1f TFLOP/s" % (lms, T / (lms * 1e-3), tf))
        result["prefill4096"] = {
            "tokens_per_s": T / (lms * 1e-3), "ms_per_call": lms, "TFLOPs": tf,
            "frac_mfma_peak": tf / MFMA_PEAK_TFLOPS, "flops_per_call": T * flops_per_token(cfg),
            "workload": "4096-token prefill, Zipf(1.1) logit bias, one layer",
        }
        del wsl

    # ---------------------------------------------------------------- CPU oracle
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(S, cfg, seed, threads)
        cb = result["cpu_baseline"]
        log("cpu oracle (%s, %d threads): decode %.2f tok/s (1 core %.2f), prefill128 %.2f tok/s (1 core %.2f)" %
            (cb["host_cpu"], threads, cb["decode_all_cores_tokens_per_s"], cb["decode_1core_tokens_per_s"],
             cb["prefill128_all_cores_tokens_per_s"], cb["prefill128_1core_tokens_per_s"]))

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

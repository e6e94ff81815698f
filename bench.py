"""Benchmark of the quantized MoE FFN layer on one MI355X.

One step = one call of the whole layer (router, top-k, routed experts,
shared expert, combine) for one decode token of a Gemma-4-26B-A4B-shaped
layer (hidden 2816, 128 experts, top-8, expert intermediate 704, shared
intermediate 2112; 8-bit router, 4-bit experts, group 64).  Calls rotate
over --layers distinct resident layers with a fresh token each, so the
256 MB Infinity Cache cannot hold the working set.  The timed calls are
replayed from a HIP graph (one capture of K calls); inputs are resident in
HBM before the timer starts.

Also reported: the 128-token prefill chunk with Zipf(1.1)-skewed routing
(same layers), and the fp64 CPU oracle timed on a bounded sample of decode
tokens.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, vendor figure
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (% of peak), decode and 128-tok prefill"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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


def decode_bytes(dev, cfg):
    """Algorithmic HBM bytes of one decode call: router, the k selected experts,
    the shared expert, the input row and the bf16 output row."""
    H, I, Is = cfg.hidden, cfg.inter, cfg.shared_inter
    import quantized_moe_gemv_amd as M
    expert = 2 * M.packed_bytes(I, H, 4) + M.packed_bytes(H, I, 4)
    shared = 2 * M.packed_bytes(Is, H, 4) + M.packed_bytes(H, Is, 4)
    router = M.packed_bytes(cfg.num_experts, H, 8)
    return router + cfg.top_k * expert + shared + 2 * H * 2, expert, router, shared


def time_graph(torch, calls, steps, warmup):
    """Capture `steps` calls in one HIP graph; warm up, then time one replay."""
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
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, g


def time_eager(torch, calls, steps):
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        calls[i % len(calls)]()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def cpu_baseline(S, cfg, seed, tokens, threads):
    import oracle as O
    host = S.make_layer(cfg, seed, layer=0)
    x = S.make_tokens(seed, tokens, cfg.hidden, batch=7)
    t0 = time.time()
    O.forward(host, x, threads=threads, dense_experts=False)
    dt = time.time() - t0
    return dict(value=tokens / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample="%d decode tokens of layer 0 (fp64 C oracle, token-parallel over %d threads), %.1f s wall"
                       % (tokens, threads, dt))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--prefill-steps", type=int, default=60)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "gemv", "grouped"])
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X and has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import qmoe_synth as S
    import quantized_moe_gemv_amd as M

    torch.cuda.set_device(0)
    cfg = S.CONFIGS["decode"]
    seed = S.SEEDS["stack30"]
    threads = min(16, os.cpu_count() or 4)
    layers = build_layers(M, S, cfg, seed, args.layers, threads)
    H, k = cfg.hidden, cfg.top_k
    per_call, expert_b, router_b, shared_b = decode_bytes(layers[0], cfg)

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
    ms, _ = time_graph(torch, calls, args.steps, args.warmup)
    ms_eager = time_eager(torch, calls, min(args.steps, 300))
    gbs = per_call / (ms * 1e-3) / 1e9
    log("decode: %.2f us/call (graph), %.2f us/call (eager), %.0f GB/s" % (ms * 1e3, ms_eager * 1e3, gbs))

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
        "data": "synthetic (seeded random 4-bit/8-bit group-64 affine codes, bf16 N(0,1) tokens)",
        "config": {
            "workload": "decode, 1 token per call, Gemma-4-26B-A4B MoE layer (H2816 E128 top8 I704 Is2112, "
                        "8-bit router, 4-bit experts, group 64), rotated over %d resident layers" % len(layers),
            "tokens_per_call": 1, "resident_layers": len(layers), "launch": "hip graph of %d calls" % args.steps,
            "weights": "int4/int8 affine group-64, bf16 scale+bias", "accumulate": "fp32", "output": "bf16",
        },
        "roofline": {
            "bound": "hbm", "kernel": "moe_layer_forward (whole call)", "achieved": gbs, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
            "bytes_per_call": per_call,
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
        pms, _ = time_graph(torch, pcalls, args.prefill_steps, max(2, args.warmup // 10))
        idh = ids.cpu().numpy()
        touched = np.array([len(np.unique(idh[i % nb])) for i in range(args.prefill_steps)])
        pbytes = router_b + touched.mean() * expert_b + shared_b + 2 * T * H * 2
        pgbs = pbytes / (pms * 1e-3) / 1e9
        log("prefill128: %.2f us/call, %.0f tokens/s, %.0f GB/s, %.1f experts touched" %
            (pms * 1e3, T / (pms * 1e-3), pgbs, touched.mean()))
        result["prefill128"] = {
            "tokens_per_s": T / (pms * 1e-3), "ms_per_call": pms, "achieved_GBs": pgbs,
            "frac_hbm_peak": pgbs / HBM_PEAK_GBS, "experts_touched_mean": float(touched.mean()),
            "bytes_per_call": float(pbytes), "calls": args.prefill_steps,
        }

    # ---------------------------------------------------------------- CPU oracle
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(S, cfg, seed, args.cpu_tokens, threads)
        log("cpu oracle: %.2f tokens/s on %d threads" % (result["cpu_baseline"]["value"], threads))

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

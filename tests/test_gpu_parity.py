"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Integer results (codes, expert ids) must match exactly; floats to the
tolerances in gpu_util.  Sizes: the tiny layer at several token counts
(several tiles and ragged tails), and the full Gemma-shaped layer at the
decode and 128-token prefill shapes, where the oracle checks every routing
decision and a sample of the outputs.
"""
import numpy as np
import pytest
import torch

import oracle as O
import qmoe_synth as S
from gpu_util import bf16_tensor, bf16_bits, check_output, check_routing, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_moe_gemv_amd as m
    return m


@pytest.fixture(scope="module")
def tiny(M):
    host = S.make_layer(S.CONFIGS["tiny"], S.SEEDS["tiny"])
    return host, M.DeviceLayer(host)


@pytest.fixture(scope="module")
def decode(M):
    host = S.make_layer(S.CONFIGS["decode"], S.SEEDS["decode"])
    return host, M.DeviceLayer(host)


@pytest.fixture(scope="module")
def prefill(M):
    host = S.make_layer(S.CONFIGS["prefill128"], S.SEEDS["prefill128"])
    return host, M.DeviceLayer(host)


@pytest.fixture(scope="module")
def large(M):
    host = S.make_layer(S.CONFIGS["prefill4096"], S.SEEDS["prefill4096"])
    return host, M.DeviceLayer(host)


def packed_dev(M, qt):
    return torch.from_numpy(M.pack(qt)).cuda()


@pytest.mark.parametrize("which", ["router", "gate", "down", "shared_gate"])
@pytest.mark.parametrize("cfg", ["tiny", "decode"])
def test_codes_and_dequant_bit_exact(M, cfg, which):
    log("codes/dequant", cfg, which)
    host = S.make_layer(S.CONFIGS[cfg], S.SEEDS[cfg])
    qt = getattr(host, which)
    if qt.codes.ndim == 3:
        qt = qt.select(3)
    buf = packed_dev(M, qt)
    codes = M.debug_unpack_codes(buf, qt.rows, qt.cols, qt.bits).cpu().numpy()
    w = M.debug_dequant(buf, qt.rows, qt.cols, qt.bits).cpu().numpy()
    if qt.rows * qt.cols <= 64 * 1024:
        assert np.array_equal(codes, O.codes(qt))
    W = O.dequant(qt)
    assert np.array_equal(w.astype(np.float64), W)        # exact: s*(q - 2^(b-1)) fits fp32
    # codes through the dequantised values: q = (w - b) / s exactly
    s = np.repeat(S.bf16_bits_to_f32(qt.scales).astype(np.float64), 64, axis=1)
    b = np.repeat(S.bf16_bits_to_f32(qt.biases).astype(np.float64), 64, axis=1)
    assert np.array_equal(codes.astype(np.float64), (W - b) / s)


@pytest.mark.parametrize("path", ["gemv", "grouped", "fused"])
@pytest.mark.parametrize("T", [1, 4, 5, 17, 40])
def test_tiny_layer(M, tiny, path, T):
    host, dev = tiny
    if path == "fused" and T > 1:
        pytest.skip("the single-launch path takes one token")
    log("tiny layer", path, "T=%d" % T)
    x = S.make_tokens(S.SEEDS["tiny"] + T, T, host.cfg.hidden)
    ref = O.forward(host, x)
    got = run_gpu(M, dev, x, path)
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    rel = check_output(ref, got, ok)
    log("  max err / RMS = %.3g" % rel)


@pytest.mark.parametrize("path", ["gemv", "grouped", "fused"])
def test_zero_input(M, tiny, path):
    host, dev = tiny
    log("zero input", path)
    T = 1 if path == "fused" else 3
    x = np.zeros((T, host.cfg.hidden), np.uint16)
    got = run_gpu(M, dev, x, path)
    k = host.cfg.top_k
    assert np.array_equal(got["ids"], np.tile(np.arange(k), (T, 1)))
    assert np.all(got["w"] == np.float32(1.0 / k))
    assert np.all(got["out32"] == 0.0) and np.all(got["out16"] == 0)


def test_tiny_zipf_and_scales(M):
    log("tiny layer with router_scale, per_expert_scale and Zipf bias")
    host = S.make_layer(S.CONFIGS["tiny"], S.SEEDS["tiny"] + 99)
    rng = np.random.default_rng(5)
    host.router_scale = rng.uniform(0.5, 1.5, host.cfg.hidden).astype(np.float32)
    host.per_expert_scale = rng.uniform(0.5, 2.0, host.cfg.num_experts).astype(np.float32)
    host.logit_bias = S.zipf_logit_bias(3, 0, host.cfg.num_experts)
    dev = M.DeviceLayer(host)
    x = S.make_tokens(77, 24, host.cfg.hidden)
    ref = O.forward(host, x)
    for path in ("gemv", "grouped"):
        got = run_gpu(M, dev, x, path)
        ok, _ = check_routing(ref, got, host.cfg.top_k)
        check_output(ref, got, ok)
    for t in (0, 5):
        got = run_gpu(M, dev, x[t:t + 1], "fused")
        sub = {key: ref[key][t:t + 1] for key in ref}
        ok, _ = check_routing(sub, got, host.cfg.top_k)
        check_output(sub, got, ok)


def test_no_shared_expert(M):
    log("tiny layer without shared expert")
    host = S.make_layer(S.CONFIGS["tiny"], S.SEEDS["tiny"] + 7, shared=False)
    dev = M.DeviceLayer(host)
    x = S.make_tokens(78, 9, host.cfg.hidden)
    ref = O.forward(host, x)
    for path in ("gemv", "grouped"):
        got = run_gpu(M, dev, x, path)
        ok, _ = check_routing(ref, got, host.cfg.top_k)
        check_output(ref, got, ok)
    got = run_gpu(M, dev, x[:1], "fused")
    sub = {key: ref[key][:1] for key in ref}
    ok, _ = check_routing(sub, got, host.cfg.top_k)
    check_output(sub, got, ok)


@pytest.mark.parametrize("T", [1, 3])
def test_decode_layer(M, decode, T):
    host, dev = decode
    log("decode layer (H2816 E128 k8 I704 Is2112)", "T=%d" % T)
    x = S.make_tokens(S.SEEDS["decode"], T, host.cfg.hidden, batch=T)
    ref = O.forward(host, x, threads=T, dense_experts=False)
    got = run_gpu(M, dev, x, "gemv")
    ok, excused = check_routing(ref, got, host.cfg.top_k)
    rel = check_output(ref, got, ok)
    log("  max err / RMS = %.3g, near-ties excused %d" % (rel, excused))
    if T == 1:
        got_f = run_gpu(M, dev, x, "fused")
        ok, _ = check_routing(ref, got_f, host.cfg.top_k)
        rel = check_output(ref, got_f, ok)
        log("  fused: max err / RMS = %.3g" % rel)
        got_a = run_gpu(M, dev, x, "auto")
        assert np.array_equal(got_a["out16"], got_f["out16"])
    else:
        got_a = run_gpu(M, dev, x, "auto")
        assert np.array_equal(got_a["out16"], got["out16"])


def test_decode_grouped_path(M, decode):
    host, dev = decode
    log("decode layer through the grouped path, T=2")
    x = S.make_tokens(S.SEEDS["decode"] + 5, 2, host.cfg.hidden)
    ref = O.forward(host, x, threads=2, dense_experts=False)
    got = run_gpu(M, dev, x, "grouped")
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    check_output(ref, got, ok)


def oracle_routing(host, x):
    """The oracle's router and top-k for every token (cheap: no experts)."""
    T = x.shape[0]
    lg = np.stack([O.router_logits(host, x[t]) for t in range(T)])
    ids = np.empty((T, host.cfg.top_k), np.int32)
    w = np.empty((T, host.cfg.top_k))
    for t in range(T):
        ids[t], w[t] = O.topk(host, lg[t])
    return dict(ids=ids, w=w, logits=lg)


def test_prefill128_layer(M, prefill):
    """The 128-token prefill chunk: every routing decision and every output
    row against the oracle."""
    host, dev = prefill
    T = 128
    log("prefill layer T=128 with Zipf routing: all 128 tokens against the oracle")
    x = S.make_tokens(S.SEEDS["prefill128"], T, host.cfg.hidden)
    got = run_gpu(M, dev, x, "auto")
    ref = O.forward(host, x, threads=16, dense_experts=False)
    ok, excused = check_routing(ref, got, host.cfg.top_k)
    counts = np.bincount(got["ids"].ravel(), minlength=host.cfg.num_experts)
    log("  experts touched %d, max tokens per expert %d, near-ties %d" % ((counts > 0).sum(), counts.max(), excused))
    rel = check_output(ref, got, ok)
    log("  max err / RMS = %.3g over %d rows" % (rel, ok.sum()))


def test_prefill4096_layer(M, large):
    """The large-batch prefill at its full size (the matrix-core regime).
    Every routing decision against the oracle's router; 256 seeded tokens, and
    every token of the experts whose whole load is one partial chunk (fewer
    than 128 tokens), against the full oracle; and every one of the 4096
    output rows against the GEMV kernels (an independent kernel family that
    the decode tests check against the oracle)."""
    host, dev = large
    T = 4096
    log("prefill layer T=4096 with Zipf routing")
    x = S.make_tokens(S.SEEDS["prefill4096"], T, host.cfg.hidden)
    got = run_gpu(M, dev, x, "auto")
    ref_r = oracle_routing(host, x)
    ok, excused = check_routing(ref_r, got, host.cfg.top_k)
    counts = np.bincount(got["ids"].ravel(), minlength=host.cfg.num_experts)
    light = [e for e in range(host.cfg.num_experts) if 0 < counts[e] < 128]
    light_tok = np.unique(np.nonzero(np.isin(got["ids"], light).any(axis=1))[0])[:160]
    sample = np.union1d(np.random.default_rng(2).choice(T, 256, replace=False), [0, T - 1])
    sample = np.union1d(sample, light_tok)
    log("  experts touched %d, max %d tokens per expert, %d experts below one chunk, near-ties %d; "
        "oracle on %d tokens" % ((counts > 0).sum(), counts.max(), len(light), excused, sample.size))
    ref = O.forward(host, x[sample], threads=16, dense_experts=False)
    sub = {key: got[key][sample] for key in ("ids", "w", "logits", "out32", "out16")}
    rel = check_output(ref, sub, ok[sample])
    log("  max err / RMS = %.3g (oracle sample)" % rel)
    gv = run_gpu(M, dev, x, "gemv")
    same = np.all(gv["ids"] == got["ids"], axis=1)
    for t in np.nonzero(~same)[0]:            # a flip between the two kernels must be an exact near-tie
        srt = np.sort(ref_r["logits"][t])[::-1]
        assert srt[host.cfg.top_k - 1] - srt[host.cfg.top_k] < 1e-5, t
    rms = np.sqrt(np.mean(gv["out32"][same] ** 2))
    err = np.max(np.abs(gv["out32"][same] - got["out32"][same]))
    log("  grouped vs GEMV kernels on %d of %d rows: max err / RMS = %.3g" % (same.sum(), T, err / rms))
    assert same.sum() >= T - 4 and err <= 1e-2 * rms


@pytest.mark.parametrize("T,chunk", [(1300, 128), (1000, 64)])
def test_midsize_layer(M, T, chunk):
    """A mid-size layer with many chunks per unit, every routing decision and
    every output row against the oracle.  Past 1024 tokens the grouped path
    runs 128-token chunks: full and partial chunks of routed and shared
    units, an odd number of 64-row tiles (the last two-tile gate/up
    workgroup has one), the down projection's four-tile workgroups, and the
    shared expert's down projection as one item over all its columns (a
    partial shared chunk too).  Up to 1024 tokens it runs 64-token chunks in
    the single GEMM launch, whose down items take the entries in the order
    their gate/up items finish (here some 60 entries, several per unit)."""
    cfg = S.LayerConfig(hidden=512, num_experts=16, inter=192, shared_inter=576, top_k=4, tokens=T, zipf=True,
                        name="mid-size layer (H512 E16 I192 Is576 k4), %d tokens, Zipf routing" % T)
    host = S.make_layer(cfg, 977)
    dev = M.DeviceLayer(host)
    log("mid-size layer T=%d on the grouped path (%d-token chunks)" % (T, chunk))
    x = S.make_tokens(978, T, cfg.hidden)
    got = run_gpu(M, dev, x, "grouped")
    ref = O.forward(host, x, threads=16, dense_experts=False)
    ok, excused = check_routing(ref, got, cfg.top_k)
    counts = np.bincount(got["ids"].ravel(), minlength=cfg.num_experts)
    log("  tokens per expert %d .. %d, near-ties %d" % (counts.min(), counts.max(), excused))
    assert (counts % chunk != 0).any() and counts.max() > chunk   # full and partial chunks
    rel = check_output(ref, got, ok)
    log("  max err / RMS = %.3g over %d rows" % (rel, ok.sum()))


def test_prefill1024_layer(M, large):
    """The Gemma-shaped layer at 1024 tokens, the largest call of the single
    GEMM launch (64-token chunks; about 250 schedule entries): every routing
    decision against the oracle's router, 128 seeded tokens against the full
    oracle, and every output row against the GEMV kernels."""
    host, dev = large
    T = 1024
    log("prefill layer T=1024 with Zipf routing (single GEMM launch)")
    x = S.make_tokens(S.SEEDS["prefill4096"] + 1, T, host.cfg.hidden)
    got = run_gpu(M, dev, x, "grouped")
    ref_r = oracle_routing(host, x)
    ok, excused = check_routing(ref_r, got, host.cfg.top_k)
    sample = np.union1d(np.random.default_rng(3).choice(T, 128, replace=False), [0, T - 1])
    ref = O.forward(host, x[sample], threads=16, dense_experts=False)
    sub = {key: got[key][sample] for key in ("ids", "w", "logits", "out32", "out16")}
    rel = check_output(ref, sub, ok[sample])
    log("  near-ties %d; max err / RMS = %.3g (oracle on %d tokens)" % (excused, rel, sample.size))
    gv = run_gpu(M, dev, x, "gemv")
    same = np.all(gv["ids"] == got["ids"], axis=1)
    for t in np.nonzero(~same)[0]:            # a flip between the two kernels must be an exact near-tie
        srt = np.sort(ref_r["logits"][t])[::-1]
        assert srt[host.cfg.top_k - 1] - srt[host.cfg.top_k] < 1e-5, t
    rms = np.sqrt(np.mean(gv["out32"][same] ** 2))
    err = np.max(np.abs(gv["out32"][same] - got["out32"][same]))
    log("  grouped vs GEMV kernels on %d of %d rows: max err / RMS = %.3g" % (same.sum(), T, err / rms))
    assert same.sum() >= T - 2 and err <= 1e-2 * rms


def test_grouped_matches_gemv_on_prefill(M, prefill):
    host, dev = prefill
    log("prefill layer T=8: grouped vs GEMV path")
    x = S.make_tokens(S.SEEDS["prefill128"] + 1, 8, host.cfg.hidden)
    a = run_gpu(M, dev, x, "gemv")
    b = run_gpu(M, dev, x, "grouped")
    assert np.array_equal(a["ids"], b["ids"])
    rms = np.sqrt(np.mean(a["out32"] ** 2))
    assert np.max(np.abs(a["out32"] - b["out32"])) <= 1e-2 * rms


@pytest.mark.parametrize("path", ["gemv", "grouped", "fused"])
def test_deterministic(M, decode, path):
    host, dev = decode
    log("determinism", path)
    x = S.make_tokens(123, 1 if path == "fused" else 6, host.cfg.hidden)
    a = run_gpu(M, dev, x, path)
    b = run_gpu(M, dev, x, path)
    assert np.array_equal(a["out32"], b["out32"]) and np.array_equal(a["ids"], b["ids"])


def test_rmsnorm(M):
    log("rmsnorm between layers")
    x = S.make_tokens(5, 7, 2816)
    want = O.rmsnorm_bf16(x, 1e-6)
    got = bf16_bits(M.rmsnorm(bf16_tensor(x), eps=1e-6))
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1 and np.count_nonzero(diff) <= x.size // 1000


@pytest.mark.parametrize("path", ["gemv", "grouped", "fused"])
def test_input_rmsnorm_in_the_call(M, tiny, path):
    """input_rmsnorm_eps > 0: the call normalises each input row first (x is
    not written).  Checked against the oracle on the normalised rows; the
    multi-launch paths normalise with the same kernel as mq_rmsnorm, so there
    the result equals normalise-then-call bit for bit."""
    host, dev = tiny
    T = 1 if path == "fused" else 6
    eps = host.cfg.eps
    log("input rmsnorm inside the call", path, "T=%d" % T)
    # rows far from unit RMS, like the output of a previous layer
    xg = bf16_tensor(S.make_tokens(S.SEEDS["tiny"] + 31, T, host.cfg.hidden)) * 37.0
    x = bf16_bits(xg)
    got = run_gpu(M, dev, x, path, input_rmsnorm_eps=eps)
    assert np.array_equal(bf16_bits(xg), x)
    ref = O.forward(host, O.rmsnorm_bf16(x, eps))
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    rel = check_output(ref, got, ok)
    log("  max err / RMS = %.3g" % rel)
    sep = run_gpu(M, dev, bf16_bits(M.rmsnorm(xg, eps=eps)), path)
    if path != "fused":
        assert np.array_equal(sep["ids"], got["ids"]) and np.array_equal(sep["out32"], got["out32"])
    with pytest.raises(M.MoeError):
        M.moe_layer_forward(dev, xg, path=path, input_rmsnorm_eps=-1.0)


def test_tiny_stack(M):
    log("4-layer tiny stack with RMS norm between layers")
    cfg = S.CONFIGS["tiny"]
    hosts = [S.make_layer(cfg, S.SEEDS["tiny"], layer=l) for l in range(4)]
    devs = [M.DeviceLayer(h) for h in hosts]
    x0 = S.make_tokens(S.SEEDS["tiny"], 2, cfg.hidden)
    xr, xg = x0, bf16_tensor(x0)
    for l, (h, d) in enumerate(zip(hosts, devs)):
        ref = O.forward(h, xr)
        ids = torch.empty((2, cfg.top_k), dtype=torch.int32, device="cuda")
        og = M.moe_layer_forward(d, xg, topk_ids=ids)
        assert np.array_equal(ids.cpu().numpy(), ref["ids"])
        if l < 3:
            xr = O.rmsnorm_bf16(ref["out_bf16"], cfg.eps)
            xg = M.rmsnorm(og, eps=cfg.eps)
    torch.cuda.synchronize()
    out = bf16_bits(og).astype(np.uint32) << 16
    outf = out.view(np.float32).astype(np.float64)
    rms = np.sqrt(np.mean(ref["out64"] ** 2))
    assert np.max(np.abs(outf - ref["out64"])) <= 1e-2 * rms + np.max(np.abs(ref["out64"])) * 2 ** -8


@pytest.mark.parametrize("path", ["gemv", "grouped", "fused"])
def test_graph_replay_matches_eager(M, tiny, path):
    host, dev = tiny
    log("hip graph replay vs eager", path)
    T = 1 if path == "fused" else 5
    xs = [bf16_tensor(S.make_tokens(900 + i, T, host.cfg.hidden)) for i in range(3)]
    ws = dev.new_workspace(5)
    eager = [M.moe_layer_forward(dev, x, workspace=ws, path=path, out_dtype=torch.float32).clone() for x in xs]
    outs = [torch.empty((T, host.cfg.hidden), dtype=torch.float32, device="cuda") for _ in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for x, o in zip(xs, outs):
                M.moe_layer_forward(dev, x, out=o, workspace=ws, path=path)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        M.moe_layer_forward(dev, xs[rep], workspace=ws, path=path)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), "replay %d differs from eager" % rep
    assert M.workspace_errors(ws) == 0


def test_fused_many_calls_interleaved(M, decode, tiny):
    """The single-launch path keeps per-workspace state across calls: run it
    many times, interleaved with the other paths and a second layer sharing
    the workspace, and check every call against the first result."""
    host, dev = decode
    log("fused path: 50 interleaved calls on one workspace")
    ws = dev.new_workspace(8)
    xa = bf16_tensor(S.make_tokens(31, 1, host.cfg.hidden))
    xb = bf16_tensor(S.make_tokens(32, 1, host.cfg.hidden))
    x8 = bf16_tensor(S.make_tokens(33, 8, host.cfg.hidden))
    ra = M.moe_layer_forward(dev, xa, workspace=ws, path="fused", out_dtype=torch.float32).clone()
    rb = M.moe_layer_forward(dev, xb, workspace=ws, path="fused", out_dtype=torch.float32).clone()
    rg = M.moe_layer_forward(dev, xa, workspace=ws, path="gemv", out_dtype=torch.float32).clone()
    for i in range(50):
        a = M.moe_layer_forward(dev, xa if i % 2 == 0 else xb, workspace=ws, path="fused", out_dtype=torch.float32)
        assert torch.equal(a, ra if i % 2 == 0 else rb), "call %d" % i
        if i % 10 == 3:
            M.moe_layer_forward(dev, x8, workspace=ws, path="grouped")
    torch.cuda.synchronize()
    assert M.workspace_errors(ws) == 0
    rms = float(torch.sqrt(torch.mean(rg.double() ** 2)))
    # the single-launch path hands the GeGLU activations to the down projection
    # as fp16 (relative rounding <= 2^-11); the GEMV path keeps 16 significant bits
    assert float(torch.max(torch.abs(ra.double() - rg.double()))) <= 4 * 2.0 ** -11 * rms


# ------------------------------------------------------------------ general affine map

GENERAL = dict(scale_range=(1e-4, 0.05), bias_range=(-0.1, 0.1))


@pytest.fixture(scope="module")
def general_decode(M):
    import dataclasses
    cfg = dataclasses.replace(S.CONFIGS["decode"], **GENERAL)
    host = S.make_layer(cfg, S.SEEDS["decode"] + 40)
    return host, M.DeviceLayer(host)


def test_general_affine_dequant(M, general_decode):
    """Independently drawn biases: the GPU's fp32 dequantised value is the
    exact s*q + b rounded once to fp32, as the oracle's exact value is."""
    host, _ = general_decode
    log("dequant with independent biases")
    for qt in (host.gate.select(5), host.shared_down):
        buf = packed_dev(M, qt)
        w = M.debug_dequant(buf, qt.rows, qt.cols, qt.bits).cpu().numpy()
        assert np.array_equal(w, O.dequant(qt).astype(np.float32))


@pytest.mark.parametrize("path", ["fused", "gemv"])
def test_general_affine_decode(M, general_decode, path):
    host, dev = general_decode
    log("decode layer, independent biases and scales U[1e-4, 0.05]:", path)
    T = 1 if path == "fused" else 3
    x = S.make_tokens(S.SEEDS["decode"] + 41, T, host.cfg.hidden, batch=T)
    ref = O.forward(host, x, threads=T, dense_experts=False)
    got = run_gpu(M, dev, x, path)
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    rel = check_output(ref, got, ok)
    log("  max err / RMS = %.3g" % rel)


def test_general_affine_prefill128(M):
    import dataclasses
    cfg = dataclasses.replace(S.CONFIGS["prefill128"], **GENERAL)
    host = S.make_layer(cfg, S.SEEDS["prefill128"] + 40)
    dev = M.DeviceLayer(host)
    log("prefill128 layer, independent biases and scales: all 128 tokens, grouped path")
    x = S.make_tokens(S.SEEDS["prefill128"] + 41, 128, cfg.hidden)
    ref = O.forward(host, x, threads=16, dense_experts=False)
    got = run_gpu(M, dev, x, "grouped")
    ok, _ = check_routing(ref, got, cfg.top_k)
    rel = check_output(ref, got, ok)
    log("  max err / RMS = %.3g" % rel)


# ------------------------------------------------------------------ input magnitude

@pytest.mark.parametrize("scale", [1e3, 1e-3])
def test_input_magnitude(M, tiny, scale):
    """Inputs far from unit RMS.  The GEMV path (bf16 pairs) matches the oracle
    at any scale; the fp16 paths match it once the call normalises its input,
    and without the norm an fp16 overflow is reported (error bit 1) with
    non-finite outputs, as the header's range precondition states."""
    host, dev = tiny
    T = 5
    log("input scaled by %g" % scale)
    xg = bf16_tensor(S.make_tokens(S.SEEDS["tiny"] + 51, T, host.cfg.hidden)) * scale
    x = bf16_bits(xg)
    ref = O.forward(host, x)
    got = run_gpu(M, dev, x, "gemv")
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    log("  gemv: max err / RMS = %.3g" % check_output(ref, got, ok))
    refn = O.forward(host, O.rmsnorm_bf16(x, host.cfg.eps))
    for path, n in (("grouped", T), ("fused", 1)):
        gn = run_gpu(M, dev, x[:n], path, input_rmsnorm_eps=host.cfg.eps)
        sub = {key: refn[key][:n] for key in refn}
        ok, _ = check_routing(sub, gn, host.cfg.top_k)
        log("  %s with the input norm: max err / RMS = %.3g" % (path, check_output(sub, gn, ok)))
    if scale > 1:
        for path, n in (("grouped", T), ("fused", 1)):
            ws = dev.new_workspace(T)
            o = M.moe_layer_forward(dev, xg[:n], workspace=ws, path=path, out_dtype=torch.float32)
            torch.cuda.synchronize()
            assert M.workspace_errors(ws) & 2, path
            assert not torch.isfinite(o).all(), path
            log("  %s without the norm: overflow reported (bit 1)" % path)


def test_give_up_reads_nan(M, tiny):
    """A wait that has given up (forced from the host by setting bit 0 of the
    workspace's error word before the call) makes the single-launch output
    NaN instead of a plausible row; a zero-filled workspace works again."""
    host, dev = tiny
    log("single-launch output after a forced give-up")
    x = bf16_tensor(S.make_tokens(S.SEEDS["tiny"] + 52, 1, host.cfg.hidden))
    ws = dev.new_workspace(1)
    good = M.moe_layer_forward(dev, x, workspace=ws, path="fused", out_dtype=torch.float32).clone()
    ws.view(torch.int32)[128] = 1          # error word: byte 512 of every workspace
    torch.cuda.synchronize()
    o = M.moe_layer_forward(dev, x, workspace=ws, path="fused", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and M.workspace_errors(ws) & 1
    ws.zero_()
    o = M.moe_layer_forward(dev, x, workspace=ws, path="fused", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, good) and M.workspace_errors(ws) == 0
    # the grouped path's single GEMM launch (down items waiting for gate/up
    # items): the same contract, with and without the layer tail
    log("grouped output after a forced give-up")
    xs = bf16_tensor(S.make_tokens(S.SEEDS["tiny"] + 53, 5, host.cfg.hidden))
    ws = dev.new_workspace(5)
    good = M.moe_layer_forward(dev, xs, workspace=ws, path="grouped", out_dtype=torch.float32).clone()
    ws.view(torch.int32)[128] = 1
    torch.cuda.synchronize()
    o = M.moe_layer_forward(dev, xs, workspace=ws, path="grouped", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and M.workspace_errors(ws) & 1
    ws.zero_()
    o = M.moe_layer_forward(dev, xs, workspace=ws, path="grouped", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, good) and M.workspace_errors(ws) == 0
    tail = M.Tail.from_dict(S.make_tail(S.SEEDS["tiny"] + 3, 0, host.cfg.hidden, norms=("shared", "routed", "out"),
                                        layer_scalar=0.75), residual_is_input=True)
    ws.view(torch.int32)[128] = 1
    torch.cuda.synchronize()
    o = M.moe_layer_forward(dev, xs, workspace=ws, path="grouped", out_dtype=torch.float32, tail=tail)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and M.workspace_errors(ws) & 1


def test_workspace_shared_across_layer_sizes(M, tiny, decode):
    """One workspace serving a small layer on the multi-launch paths and then
    the Gemma-shaped layer on the single-launch path: the small layer's
    buffers must not land on the words the single-launch path keeps across
    calls (regression: they did, and a stale word equal to the next tag was
    taken as current)."""
    th, td = tiny
    dh, dd = decode
    log("one workspace: tiny layer (gemv, grouped) then the decode layer (fused)")
    ws = torch.zeros(max(td.workspace_bytes(40), dd.workspace_bytes(1)), dtype=torch.uint8, device="cuda")
    xd = bf16_tensor(S.make_tokens(S.SEEDS["decode"] + 70, 1, dh.cfg.hidden))
    want = M.moe_layer_forward(dd, xd, path="fused", out_dtype=torch.float32)
    for i in range(3):
        for path, T in (("gemv", 4), ("grouped", 40), ("fused", 1)):
            xt = bf16_tensor(S.make_tokens(S.SEEDS["tiny"] + 70 + i, T, th.cfg.hidden))
            M.moe_layer_forward(td, xt, workspace=ws, path=path)
        got = M.moe_layer_forward(dd, xd, workspace=ws, path="fused", out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, want), "round %d" % i
    assert M.workspace_errors(ws) == 0

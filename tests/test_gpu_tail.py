"""The layer tail (post-FFN norms, residual, layer scalar) on every path,
through the C ABI, against the oracle's oq_moe_forward_ex: ids exact, the
fp32 output within 1e-2 of the exact output's RMS, the bf16 output its
single rounding.  Also one token through a stack of layers with tails in
one launch, bit for bit the chained single-launch calls."""
import numpy as np
import pytest
import torch

import oracle as O
import qmoe_synth as S
from gpu_util import bf16_bits, bf16_tensor, check_output, check_routing, log, run_gpu

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


NORM_SETS = {
    "all": ("shared", "routed", "out"),
    "branches": ("shared", "routed"),
    "out_only": ("out",),
    "none": (),
}


@pytest.mark.parametrize("norms", list(NORM_SETS))
@pytest.mark.parametrize("path,T", [("gemv", 4), ("grouped", 40), ("fused", 1)])
def test_tail_paths(M, tiny, path, T, norms):
    host, dev = tiny
    H = host.cfg.hidden
    log("tail", norms, path, "T=%d" % T)
    t = S.make_tail(S.SEEDS["tiny"] + 3, 0, H, norms=NORM_SETS[norms], layer_scalar=0.75)
    x = S.make_tokens(S.SEEDS["tiny"] + 80, T, H)
    # residual = the input rows themselves
    ref = O.forward(host, x, tail=t, resid=x)
    got = run_gpu(M, dev, x, path, tail=M.Tail.from_dict(t, residual_is_input=True))
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    log("  residual = input: max err / RMS = %.3g" % check_output(ref, got, ok))
    # an explicit residual, and the input normalised inside the call while the
    # residual stays the given rows
    res = S.make_tokens(S.SEEDS["tiny"] + 81, T, H)
    ref = O.forward(host, x, tail=t, resid=res)
    got = run_gpu(M, dev, x, path, tail=M.Tail.from_dict(t, residual=bf16_tensor(res)))
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    log("  explicit residual: max err / RMS = %.3g" % check_output(ref, got, ok))
    xs = bf16_bits(bf16_tensor(x) * 5.0)
    ref = O.forward(host, O.rmsnorm_bf16(xs, host.cfg.eps), tail=t, resid=xs)
    got = run_gpu(M, dev, xs, path, input_rmsnorm_eps=host.cfg.eps, tail=M.Tail.from_dict(t, residual_is_input=True))
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    log("  normalised input, residual = input as given: max err / RMS = %.3g" % check_output(ref, got, ok))


@pytest.mark.parametrize("path,T", [("fused", 1), ("gemv", 2), ("grouped", 24)])
def test_tail_decode_layer(M, path, T):
    cfg = S.CONFIGS["decode"]
    host = S.make_layer(cfg, S.SEEDS["decode"])
    dev = M.DeviceLayer(host)
    log("tail on the decode layer", path, "T=%d" % T)
    t = S.make_tail(S.SEEDS["decode"] + 3, 0, cfg.hidden, layer_scalar=1.25)
    x = S.make_tokens(S.SEEDS["decode"] + 82, T, cfg.hidden)
    ref = O.forward(host, x, threads=min(T, 16), dense_experts=False, tail=t, resid=x)
    got = run_gpu(M, dev, x, path, tail=M.Tail.from_dict(t, residual_is_input=True))
    ok, _ = check_routing(ref, got, cfg.top_k)
    log("  max err / RMS = %.3g" % check_output(ref, got, ok))


def test_tail_stack_equals_chained_calls(M):
    """Three layers with tails in one launch: layer l's residual is its input
    (the previous layer's output), its experts see that input normalised.
    Bit for bit the chained single-launch calls, and each layer within the
    tolerance of the oracle fed the same input row as the GPU layer."""
    cfg = S.CONFIGS["tiny"]
    hosts = [S.make_layer(cfg, S.SEEDS["tiny"] + 5, layer=l) for l in range(3)]
    devs = [M.DeviceLayer(h) for h in hosts]
    tails = [S.make_tail(S.SEEDS["tiny"] + 6, l, cfg.hidden, layer_scalar=0.5 + 0.25 * l) for l in range(3)]
    dt = [M.Tail.from_dict(t, residual_is_input=True) for t in tails]
    log("3-layer stack with tails")
    x = S.make_tokens(S.SEEDS["tiny"] + 83, 1, cfg.hidden)
    xg = bf16_tensor(x)
    st = M.Stack(devs)
    ids = torch.empty((3, cfg.top_k), dtype=torch.int32, device="cuda")
    got = M.moe_stack_forward(st, xg, between_eps=cfg.eps, out_dtype=torch.float32, tails=dt, topk_ids=ids)
    cur = xg
    for l in range(3):
        xin = bf16_bits(cur)
        kw = dict(path="fused", input_rmsnorm_eps=0.0 if l == 0 else cfg.eps, tail=dt[l])
        o32 = M.moe_layer_forward(devs[l], cur, out_dtype=torch.float32, **kw)
        if l < 2:
            cur = M.moe_layer_forward(devs[l], cur, out_dtype=torch.bfloat16, **kw)
        torch.cuda.synchronize()
        # this layer against the oracle fed the same (GPU) input row
        ref = O.forward(hosts[l], xin if l == 0 else O.rmsnorm_bf16(xin, cfg.eps), tail=tails[l], resid=xin)
        assert np.array_equal(ids.cpu().numpy()[l], ref["ids"][0]), l
        rms = np.sqrt(np.mean(ref["out64"] ** 2))
        err = np.max(np.abs(o32.cpu().numpy().astype(np.float64) - ref["out64"]))
        log("  layer %d: max err / RMS = %.3g" % (l, err / rms))
        assert err <= 1e-2 * rms
    assert torch.equal(got, o32)


def test_tail_prefill128_all_rows(M):
    cfg = S.CONFIGS["prefill128"]
    host = S.make_layer(cfg, S.SEEDS["prefill128"])
    dev = M.DeviceLayer(host)
    log("tail on the prefill128 layer, all 128 rows")
    t = S.make_tail(S.SEEDS["prefill128"] + 3, 0, cfg.hidden)
    x = S.make_tokens(S.SEEDS["prefill128"] + 84, 128, cfg.hidden)
    ref = O.forward(host, x, threads=16, dense_experts=False, tail=t, resid=x)
    got = run_gpu(M, dev, x, "grouped", tail=M.Tail.from_dict(t, residual_is_input=True))
    ok, _ = check_routing(ref, got, cfg.top_k)
    log("  max err / RMS = %.3g" % check_output(ref, got, ok))

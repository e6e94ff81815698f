"""GPU parity of the single-launch stack (moe_stack_forward): one token
through several layers in one launch, with the unit-weight RMS norm between
layers.  Checked against the fp64 oracle chained the same way (every
layer's expert ids exact, the last output to the float bar) and, bit for
bit, against the same layers run as separate single-launch calls.
"""
import numpy as np
import pytest
import torch

import oracle as O
import qmoe_synth as S
from gpu_util import REL_TOL, bf16_bits, bf16_half_ulp, bf16_tensor, bf16_to_f64, check_routing, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_moe_gemv_amd as m
    return m


def tiny_hosts(n, scales=False):
    cfg = S.CONFIGS["tiny"]
    hosts = [S.make_layer(cfg, S.SEEDS["tiny"], layer=l) for l in range(n)]
    if scales:
        rng = np.random.default_rng(17)
        for l, h in enumerate(hosts):
            h.router_scale = rng.uniform(0.5, 1.5, cfg.hidden).astype(np.float32)
            h.per_expert_scale = rng.uniform(0.5, 2.0, cfg.num_experts).astype(np.float32)
            h.logit_bias = S.zipf_logit_bias(3 + l, l, cfg.num_experts)
    return hosts


def chained_calls(M, devs, x, eps, out_dtype, ins=None):
    """The same stack as separate single-launch calls; per-layer ids, weights,
    scores, and (into `ins`) each layer's input row."""
    k, E = devs[0].top_k, devs[0].num_experts
    ids = torch.empty((len(devs), k), dtype=torch.int32, device="cuda")
    w = torch.empty((len(devs), k), dtype=torch.float32, device="cuda")
    lg = torch.empty((len(devs), E), dtype=torch.float32, device="cuda")
    cur = x
    ws = devs[0].new_workspace(1)
    for l, d in enumerate(devs):
        if ins is not None:
            ins.append(cur)
        last = l == len(devs) - 1
        cur = M.moe_layer_forward(d, cur, workspace=ws, path="fused", out_dtype=out_dtype if last else torch.bfloat16,
                                  topk_ids=ids[l:l + 1], topk_w=w[l:l + 1], logits=lg[l:l + 1],
                                  input_rmsnorm_eps=eps if l > 0 else 0.0)
    torch.cuda.synchronize()
    assert M.workspace_errors(ws) == 0
    return cur, ids, w, lg


def stack_call(M, stack, x, eps, out_dtype, ws=None):
    n, k, E = len(stack), stack.top_k, stack.num_experts
    ids = torch.full((n, k), -1, dtype=torch.int32, device="cuda")
    w = torch.empty((n, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((n, E), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = stack.new_workspace()
    out = M.moe_stack_forward(stack, x, workspace=ws, between_eps=eps, out_dtype=out_dtype, topk_ids=ids, topk_w=w,
                              logits=lg)
    torch.cuda.synchronize()
    assert M.workspace_errors(ws) == 0, "a bounded wait of the single-launch stack gave up"
    return out, ids, w, lg


@pytest.mark.parametrize("scales", [False, True])
@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_tiny_stack_against_oracle_and_chained_calls(M, scales, eps):
    # Without the norm between layers a row shrinks about quadratically per
    # layer (GeGLU of a small input); by the third layer the activations fall
    # below fp16's normal range, where the fp16 activation rows of the
    # single-launch path lose precision.  Two layers cover the hand-off.
    n = 5 if eps > 0 else 2
    log("single-launch stack of %d tiny layers" % n, "scales" if scales else "", "eps=%g" % eps)
    hosts = tiny_hosts(n, scales)
    devs = [M.DeviceLayer(h) for h in hosts]
    stack = M.Stack(devs)
    cfg = hosts[0].cfg
    x0 = S.make_tokens(S.SEEDS["tiny"] + 7, 1, cfg.hidden)
    x = bf16_tensor(x0)
    for out_dtype in (torch.float32, torch.bfloat16):
        got, ids, w, lg = stack_call(M, stack, x, eps, out_dtype)
        ins = []
        want, ids_c, w_c, lg_c = chained_calls(M, devs, x, eps, out_dtype, ins)
        assert torch.equal(ids, ids_c) and torch.equal(w, w_c) and torch.equal(lg, lg_c)
        assert torch.equal(got, want), "stack differs from the chained single-layer calls"
    assert np.array_equal(bf16_bits(x), x0)          # the input is not written
    # every layer against the oracle on the same input row (normalised by the
    # oracle's own RMS norm): routing exact, output to the float bar
    outs = ins[1:] + [got]
    for l, h in enumerate(hosts):
        xin = bf16_bits(ins[l])
        if l > 0 and eps > 0:
            xin = O.rmsnorm_bf16(xin, eps)
        ref = O.forward(h, xin)
        gl = dict(ids=ids[l:l + 1].cpu().numpy(), w=w[l:l + 1].cpu().numpy(), logits=lg[l:l + 1].cpu().numpy())
        ok, _ = check_routing(ref, gl, cfg.top_k)
        if ok.all():
            r64 = ref["out64"]
            o16 = bf16_to_f64(bf16_bits(outs[l]))
            rms = np.sqrt(np.mean(r64 ** 2))
            assert np.all(np.abs(o16 - r64) <= REL_TOL * rms + bf16_half_ulp(r64) * 1.0001), "layer %d output" % l


def test_one_layer_stack_equals_the_layer_call(M):
    log("a stack of one layer is the single-launch layer call")
    hosts = tiny_hosts(1)
    dev = M.DeviceLayer(hosts[0])
    x = bf16_tensor(S.make_tokens(71, 1, hosts[0].cfg.hidden)) * 3.0
    st = M.Stack([dev])
    for in_eps in (0.0, 1e-6):
        ws = st.new_workspace()
        got = M.moe_stack_forward(st, x, workspace=ws, input_rmsnorm_eps=in_eps, out_dtype=torch.float32)
        want = M.moe_layer_forward(dev, x, path="fused", input_rmsnorm_eps=in_eps, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, want)


@pytest.fixture(scope="module")
def decode_stack(M):
    cfg = S.CONFIGS["decode"]
    hosts = [S.make_layer(cfg, S.SEEDS["stack30"], layer=l) for l in range(3)]
    devs = [M.DeviceLayer(h) for h in hosts]
    return hosts, devs


def test_decode_stack_matches_chained_calls(M, decode_stack):
    hosts, devs = decode_stack
    log("single-launch stack of 3 decode-shaped layers")
    stack = M.Stack(devs)
    cfg = hosts[0].cfg
    x0 = S.make_tokens(S.SEEDS["stack30"] + 1, 1, cfg.hidden)
    x = bf16_tensor(x0)
    got, ids, w, lg = stack_call(M, stack, x, cfg.eps, torch.float32)
    want, ids_c, w_c, lg_c = chained_calls(M, devs, x, cfg.eps, torch.float32)
    assert torch.equal(ids, ids_c) and torch.equal(w, w_c) and torch.equal(lg, lg_c)
    assert torch.equal(got, want)
    # the first layer's routing against the oracle (its input is the caller's x)
    ref = O.forward(hosts[0], x0)
    assert np.array_equal(ids[0].cpu().numpy(), ref["ids"][0])
    assert np.allclose(w[0].cpu().numpy(), ref["w"][0], rtol=0, atol=1e-5)


def test_stack_graph_replay_and_shared_workspace(M, decode_stack):
    """Replays of a captured stack call, with single-layer calls on the same
    workspace between them, give the eager result every time."""
    hosts, devs = decode_stack
    log("stack: graph replay, interleaved with layer calls on one workspace")
    stack = M.Stack(devs)
    cfg = hosts[0].cfg
    ws = stack.new_workspace()
    assert ws.numel() >= devs[0].workspace_bytes(1)
    xs = [bf16_tensor(S.make_tokens(500 + i, 1, cfg.hidden)) for i in range(2)]
    eager = [M.moe_stack_forward(stack, x, workspace=ws, between_eps=cfg.eps, out_dtype=torch.float32).clone()
             for x in xs]
    lay = M.moe_layer_forward(devs[1], xs[0], workspace=ws, path="fused", out_dtype=torch.float32).clone()
    outs = [torch.empty((1, cfg.hidden), dtype=torch.float32, device="cuda") for _ in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for x, o in zip(xs, outs):
                M.moe_stack_forward(stack, x, out=o, workspace=ws, between_eps=cfg.eps)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        l2 = M.moe_layer_forward(devs[1], xs[0], workspace=ws, path="fused", out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(l2, lay)
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), "replay %d differs from eager" % rep
    assert M.workspace_errors(ws) == 0

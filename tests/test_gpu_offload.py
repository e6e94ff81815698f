"""The host-offloaded expert pool, through the C ABI: routing only
(mq_route) equals the routing of a layer call; a layer call with the routing
given equals the call that routes itself, bit for bit; and an OffloadedLayer
(experts in pinned host memory, 16 device slots under the LFU cache, copies
on a second stream, the shared expert before the wait for them) gives, token
after token, the same outputs as the same layer resident in HBM, and the
oracle's within the tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
import qmoe_synth as S
from gpu_util import bf16_bits, bf16_tensor, check_output, check_routing, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_moe_gemv_amd as m
    return m


@pytest.fixture(scope="module")
def decode(M):
    host = S.make_layer(S.CONFIGS["decode"], S.SEEDS["decode"] + 200)
    host.logit_bias = S.zipf_logit_bias(S.SEEDS["decode"] + 200, 0, host.cfg.num_experts)
    return host, M.DeviceLayer(host)


def test_route_equals_the_layer_calls_routing(M, decode):
    host, dev = decode
    log("mq_route vs the GEMV path's own routing")
    x = bf16_tensor(S.make_tokens(201, 4, host.cfg.hidden))
    ids, w = M.route(dev, x)
    ids2 = torch.empty_like(ids)
    w2 = torch.empty_like(w)
    M.moe_layer_forward(dev, x, path="gemv", topk_ids=ids2, topk_w=w2)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2)


@pytest.mark.parametrize("T", [1, 4])
def test_given_routing_equals_the_routed_call(M, decode, T):
    host, dev = decode
    log("given routing, T=%d" % T)
    x = bf16_tensor(S.make_tokens(202 + T, T, host.cfg.hidden))
    a = M.moe_layer_forward(dev, x, path="gemv", out_dtype=torch.float32)
    ids, w = M.route(dev, x)
    b = M.moe_layer_forward(dev, x, out_dtype=torch.float32, route_ids=ids, route_w=w)
    ev = torch.cuda.Event()
    ev.record()
    c = M.moe_layer_forward(dev, x, out_dtype=torch.float32, route_ids=ids, route_w=w, experts_ready=ev)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    with pytest.raises(M.MoeError):
        M.moe_layer_forward(dev, x, path="grouped", route_ids=ids, route_w=w)


def test_offloaded_layer_token_sequence(M, decode):
    host, dev = decode
    off = M.OffloadedLayer(host, num_slots=16)
    log("offloaded experts, 16 slots: 48 decode tokens (Zipf-skewed routing) against the resident layer")
    x = S.make_tokens(210, 48, host.cfg.hidden)
    xg = bf16_tensor(x)
    for t in range(48):
        got = off.forward(xg[t:t + 1], out_dtype=torch.float32)
        want = M.moe_layer_forward(dev, xg[t:t + 1], path="gemv", out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, want), t
    log("  hits %d, misses %d" % (off.hits, off.misses))
    assert off.misses >= 16 and off.hits > 0
    # a few tokens against the oracle, and a 4-token call
    for t in (0, 47):
        ref = O.forward(host, x[t:t + 1], dense_experts=False)
        o = off.forward(xg[t:t + 1], out_dtype=torch.float32)
        o16 = off.forward(xg[t:t + 1])
        torch.cuda.synchronize()
        got = dict(ids=ref["ids"], w=ref["w"], logits=ref["logits"], out32=o.cpu().numpy().astype(np.float64),
                   out16=bf16_bits(o16))
        log("  token %d: max err / RMS = %.3g" % (t, check_output(ref, got)))
    # two tokens (at most 16 distinct experts: they always fit the slots)
    o2 = off.forward(xg[:2], out_dtype=torch.float32)
    w2 = M.moe_layer_forward(dev, xg[:2], path="gemv", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o2, w2)
    # more distinct experts than slots: refused before anything is enqueued
    ids4, _ = M.route(dev, xg[:4])
    if len(set(ids4.cpu().numpy().ravel().tolist())) > 16:
        with pytest.raises(M.MoeError) as e:
            off.forward(xg[:4])
        assert e.value.status == M.MQ_ERR_SHAPE


def test_offloaded_layer_with_tail_and_input_norm(M, decode):
    host, dev = decode
    off = M.OffloadedLayer(host, num_slots=16)
    t = S.make_tail(5, 0, host.cfg.hidden)
    tl = M.Tail.from_dict(t, residual_is_input=True)
    log("offloaded experts with the layer tail and the input norm")
    xg = bf16_tensor(S.make_tokens(220, 3, host.cfg.hidden)) * 4.0
    for i in range(3):
        got = off.forward(xg[i:i + 1], out_dtype=torch.float32, tail=tl, input_rmsnorm_eps=1e-6)
        want = M.moe_layer_forward(dev, xg[i:i + 1], path="gemv", out_dtype=torch.float32, tail=tl,
                                   input_rmsnorm_eps=1e-6)
        torch.cuda.synchronize()
        assert torch.equal(got, want), i

"""Other widths of the affine format against the oracle, through the C ABI:
8-bit routed and shared experts (run by the GEMV kernels at any token
count), and a group size of 128 (packed into the group-64 device layout
with each pair repeated, run by every path).  Same bar as the 4-bit layer:
ids exact, fp32 output within 1e-2 of the exact output's RMS, bf16 output
its single rounding; dequantised values bit-exact (fp32 of the exact s q + b)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import qmoe_synth as S
from gpu_util import check_output, check_routing, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_moe_gemv_amd as m
    return m


def layer(M, name, seed_off, **kw):
    cfg = dataclasses.replace(S.CONFIGS[name], **kw)
    host = S.make_layer(cfg, S.SEEDS[name] + seed_off)
    return host, M.DeviceLayer(host)


GEN8 = dict(expert_bits=8, scale_range=(2e-4, 2e-3), bias_range=(-0.1, 0.1))


@pytest.fixture(scope="module")
def tiny8(M):
    return layer(M, "tiny", 100, **GEN8)


def test_8bit_dequant_bit_exact(M, tiny8):
    host, _ = tiny8
    for qt in (host.gate.select(3), host.down.select(7), host.shared_up):
        assert qt.bits == 8
        buf = torch.from_numpy(M.pack(qt)).cuda()
        codes = M.debug_unpack_codes(buf, qt.rows, qt.cols, 8).cpu().numpy()
        w = M.debug_dequant(buf, qt.rows, qt.cols, 8).cpu().numpy()
        assert np.array_equal(codes, O.codes(qt))
        assert np.array_equal(w, O.dequant(qt).astype(np.float32))


@pytest.mark.parametrize("T", [1, 4, 40])
def test_8bit_experts_tiny(M, tiny8, T):
    host, dev = tiny8
    log("8-bit experts, tiny layer, T=%d" % T)
    x = S.make_tokens(S.SEEDS["tiny"] + 101 + T, T, host.cfg.hidden)
    ref = O.forward(host, x)
    got = run_gpu(M, dev, x, "auto")
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    log("  max err / RMS = %.3g" % check_output(ref, got, ok))
    with pytest.raises(M.MoeError):
        M.moe_layer_forward(dev, torch.zeros((T, host.cfg.hidden), dtype=torch.bfloat16, device="cuda"),
                            path="grouped")


def test_8bit_experts_with_tail(M, tiny8):
    host, dev = tiny8
    log("8-bit experts with the layer tail")
    x = S.make_tokens(S.SEEDS["tiny"] + 120, 3, host.cfg.hidden)
    t = S.make_tail(7, 0, host.cfg.hidden)
    ref = O.forward(host, x, tail=t, resid=x)
    got = run_gpu(M, dev, x, "auto", tail=M.Tail.from_dict(t, residual_is_input=True))
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    log("  max err / RMS = %.3g" % check_output(ref, got, ok))


@pytest.mark.parametrize("T", [1, 3])
def test_8bit_experts_decode_shape(M, T):
    host, dev = layer(M, "decode", 100, **GEN8)
    log("8-bit experts, decode layer (H2816 E128 I704 Is2112), T=%d" % T)
    x = S.make_tokens(S.SEEDS["decode"] + 102, T, host.cfg.hidden, batch=T)
    ref = O.forward(host, x, threads=T, dense_experts=False)
    got = run_gpu(M, dev, x, "auto")
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    log("  max err / RMS = %.3g" % check_output(ref, got, ok))


@pytest.mark.parametrize("path,T", [("fused", 1), ("gemv", 4), ("grouped", 40)])
def test_group128(M, path, T):
    # every matrix width (256, 128, 256) a multiple of the group
    host, dev = layer(M, "tiny", 110, group=128, inter=128, shared_inter=256, bias_range=(-0.05, 0.05))
    assert host.gate.group == 128 and host.gate.scales.shape[-1] == host.cfg.hidden // 128
    log("group 128, tiny layer", path, "T=%d" % T)
    x = S.make_tokens(S.SEEDS["tiny"] + 111 + T, T, host.cfg.hidden)
    ref = O.forward(host, x)
    got = run_gpu(M, dev, x, path)
    ok, _ = check_routing(ref, got, host.cfg.top_k)
    log("  max err / RMS = %.3g" % check_output(ref, got, ok))

"""The allocation-free entry point (moe_layer_forward_noalloc) against the
workspace entry point, through the C ABI: the same kernels on the library's
fixed device scratch must give the same results, bit for bit, on two calls
in a row with the second smaller, on every path; and a call too large for
the scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

import qmoe_synth as S
from gpu_util import bf16_tensor, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_moe_gemv_amd as m
    return m


def both(M, dev, x, path):
    T = x.shape[0]
    ids_a = torch.empty((T, dev.top_k), dtype=torch.int32, device="cuda")
    ids_b = torch.empty_like(ids_a)
    ws = dev.new_workspace(T)
    a = M.moe_layer_forward(dev, x, workspace=ws, path=path, out_dtype=torch.float32, topk_ids=ids_a)
    out = torch.full((T, dev.hidden), float("nan"), dtype=torch.float32, device="cuda")
    b = M.moe_layer_forward_noalloc(dev, x, out=out, path=path, topk_ids=ids_b)
    torch.cuda.synchronize()
    assert M.workspace_errors(ws) == 0
    return a, b, ids_a, ids_b


@pytest.mark.parametrize("cfg,path,sizes", [
    ("tiny", "fused", (1, 1)),
    ("tiny", "gemv", (4, 2)),
    ("tiny", "grouped", (40, 6)),
    ("decode", "fused", (1, 1)),
    ("decode", "auto", (128, 16)),
])
def test_noalloc_matches_workspace_entry(M, cfg, path, sizes):
    host = S.make_layer(S.CONFIGS[cfg], S.SEEDS[cfg])
    dev = M.DeviceLayer(host)
    for i, T in enumerate(sizes):
        log("noalloc vs workspace entry:", cfg, path, "T=%d" % T)
        x = bf16_tensor(S.make_tokens(S.SEEDS[cfg] + 60 + i, T, host.cfg.hidden))
        a, b, ia, ib = both(M, dev, x, path)
        assert torch.equal(ia, ib)
        assert torch.equal(a, b), "call %d (T=%d) differs" % (i, T)


def test_noalloc_refuses_calls_beyond_the_scratch(M):
    host = S.make_layer(S.CONFIGS["decode"], S.SEEDS["decode"], experts=True)
    dev = M.DeviceLayer(host)
    assert M.noalloc_scratch_bytes() == 40 << 20
    assert dev.workspace_bytes(128) <= M.noalloc_scratch_bytes() < dev.workspace_bytes(256)
    x = bf16_tensor(S.make_tokens(5, 256, host.cfg.hidden))
    out = torch.zeros((256, host.cfg.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoeError) as e:
        M.moe_layer_forward_noalloc(dev, x, out=out)
    assert e.value.status == M.MQ_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0

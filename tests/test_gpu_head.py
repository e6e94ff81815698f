"""The quantized GEMV head (mq_qgemv) against the oracle's oq_qgemv_head:
the tied 4-bit head at its full synthetic size (262,144 rows x 2816) with the
final softcap 30 and the greedy argmax, and small ragged shapes (rows not a
multiple of 64, several tokens, 4- and 8-bit codes, with and without the
cap).  Logits within 1e-2 of the exact logits' RMS (bf16 logits the single
rounding of the fp32 ones); argmax exact unless the exact top two are
closer than 1e-5."""
import numpy as np
import pytest
import torch

import oracle as O
import qmoe_synth as S
from gpu_util import bf16_bits, bf16_tensor, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_moe_gemv_amd as m
    return m


def check(ref_lg, ref_am, y, am, tol=1e-2):
    rms = np.sqrt(np.mean(ref_lg ** 2))
    err = np.max(np.abs(y.astype(np.float64) - ref_lg))
    assert err <= tol * rms, (err, rms)
    for t in range(ref_lg.shape[0]):
        if am[t] != ref_am[t]:
            top = np.sort(ref_lg[t])[::-1]
            assert top[0] - top[1] < 1e-5 and ref_lg[t][am[t]] >= top[0] - 1e-5, t
    return err / rms


def test_head_full_vocab(M):
    V, H = S.HEAD_VOCAB, S.CONFIGS["decode"].hidden
    log("head %d x %d, 4-bit, softcap 30, one token" % (V, H))
    qt = S.make_head(S.SEEDS["decode"] + 90, V, H)
    buf = torch.from_numpy(M.pack(qt)).cuda()
    x = S.make_tokens(S.SEEDS["decode"] + 91, 1, H)
    y, am = M.qgemv(buf, V, H, 4, bf16_tensor(x), softcap=30.0)
    torch.cuda.synchronize()
    ref_lg, ref_am = O.qgemv_head(qt, x, 30.0)
    rel = check(ref_lg, ref_am, y.cpu().numpy(), am.cpu().numpy())
    log("  max err / RMS = %.3g, argmax %d (oracle %d)" % (rel, am.cpu().item(), ref_am[0]))
    _, am2 = M.qgemv(buf, V, H, 4, bf16_tensor(x), softcap=30.0, want_y=False)
    assert torch.equal(am2, am)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("cap", [0.0, 5.0])
@pytest.mark.parametrize("V,H,T", [(1000, 256, 3), (64, 128, 1), (4097, 512, 8)])
def test_head_small_shapes(M, bits, cap, V, H, T):
    log("head %d x %d, %d-bit, cap %g, T=%d" % (V, H, bits, cap, T))
    # scales keeping the logits within a few units, where tanh(y / 5) still responds
    lo, hi = (0.005, 0.03) if bits == 4 else (0.0003, 0.002)
    qt = S.make_qtensor(77 + V, 0, 0, S.T_HEAD_CODES, S.T_HEAD_SCALES, V, H, bits, scale_lo=lo, scale_hi=hi,
                        bias_range=(-0.05, 0.05))
    buf = torch.from_numpy(M.pack(qt)).cuda()
    x = S.make_tokens(78 + V, T, H)
    y, am = M.qgemv(buf, V, H, bits, bf16_tensor(x), softcap=cap)
    yb, amb = M.qgemv(buf, V, H, bits, bf16_tensor(x), softcap=cap, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref_lg, ref_am = O.qgemv_head(qt, x, cap)
    check(ref_lg, ref_am, y.cpu().numpy(), am.cpu().numpy())
    assert torch.equal(am, amb)
    assert np.array_equal(bf16_bits(yb), bf16_bits(y.to(torch.bfloat16)))
    if cap > 0:
        assert float(y.abs().max()) <= cap
        assert float(y.abs().max()) > 0.25 * cap    # the cap was exercised


def test_head_argmax_ties_go_to_the_lower_row(M):
    V, H = 300, 128
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(V, H)).astype(np.uint32)
    q[250] = q[70] = 15                               # two identical rows, far above the rest
    lo, hi = q[:, 0::2].astype(np.uint8), q[:, 1::2].astype(np.uint8)
    codes = (lo | (hi << 4)).astype(np.uint8).copy().view("<u4")
    sc = np.full((V, H // 64), 0x3C00, np.uint16)     # bf16 0.0078125
    bi = np.zeros((V, H // 64), np.uint16)
    qt = S.QTensor(np.ascontiguousarray(codes), sc, bi, V, H, 4)
    buf = torch.from_numpy(M.pack(qt)).cuda()
    x = bf16_tensor(np.full((2, H), 0x3F80, np.uint16))
    _, am = M.qgemv(buf, V, H, 4, x, softcap=30.0, want_y=False)
    assert am.cpu().tolist() == [70, 70]
    assert O.qgemv_head(qt, bf16_bits(x), 30.0)[1].tolist() == [70, 70]

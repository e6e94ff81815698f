"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against one of: values printed on the pages
(tests/golden/), closed forms, special cases that reduce to a library
routine (torch's bf16 cast and tanh-GELU, numpy matmul, scipy's softmax),
invariants of the method, or brute force.  ``test_planted_mistakes_are_caught``
rebuilds the oracle with single planted mistakes and checks that this file
catches every one of them.
"""
import os
import re
import shutil
import tempfile

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
import qmoe_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def page_constants():
    out = {}
    with open(os.path.join(GOLDEN, "page_constants.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = int(v)
    return out


def f32_to_bf16_bits(v):
    """bf16 bit patterns through torch's cast (round to nearest even)."""
    t = torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def bf16_bits_to_f64(b):
    return torch.tensor(np.asarray(b, dtype=np.uint16).astype(np.int16)).view(torch.bfloat16).double().numpy()


def qtensor_from_codes(q, scales, biases, bits):
    """Pack an integer code matrix q [rows][cols] into canonical words through a
    byte view (a route independent of the oracle's word shifts)."""
    q = np.asarray(q, dtype=np.uint32)
    rows, cols = q.shape
    if bits == 8:
        words = q.astype(np.uint8).reshape(rows, cols).copy().view("<u4")
    else:
        lo = q[:, 0::2].astype(np.uint8)
        hi = q[:, 1::2].astype(np.uint8)
        words = (lo | (hi << 4)).astype(np.uint8).copy().view("<u4")
    return S.QTensor(np.ascontiguousarray(words), np.asarray(scales, np.uint16),
                     np.asarray(biases, np.uint16), rows, cols, bits)


def tiny_layer(seed=S.SEEDS["tiny"]):
    return S.make_layer(S.CONFIGS["tiny"], seed)


def tiny_tokens(seed=S.SEEDS["tiny"], T=4):
    return S.make_tokens(seed, T, S.CONFIGS["tiny"].hidden)


# ------------------------------------------------------------------ pages

def test_page_constants_match_workload_shapes():
    pc = page_constants()
    cfg = S.CONFIGS["decode"]
    assert cfg.num_experts == pc["num_experts"] and cfg.top_k == pc["top_k"]
    assert S.GROUP == pc["group_size"]
    H, I = cfg.hidden, cfg.inter
    # one routed expert: gate [I][H] + up [I][H] + down [H][I], 4-bit codes, bf16 scale+bias per 64
    per_matrix = I * H * pc["expert_bits"] // 8 + (I * H // pc["group_size"]) * 4
    blob = 3 * per_matrix
    page = pc["page_bytes"]
    rounded = (blob + page - 1) // page * page
    assert rounded == pc["page_rounded_expert_blob_bytes"]
    assert pc["num_layers"] * cfg.num_experts * rounded == pc["routed_expert_files_bytes"]


# ------------------------------------------------------------------ bf16

def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, 2.0 ** -130]]).astype(np.float32)
    want = f32_to_bf16_bits(v)
    got = np.array([O.bf16_round(float(x)) for x in v], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_round_halfway_cases():
    assert O.bf16_round(1.0) == 0x3F80
    assert O.bf16_round(1.0 + 2 ** -8) == 0x3F80          # tie -> even (down)
    assert O.bf16_round(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert O.bf16_round(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81  # just above the tie: rounds once from fp64
    assert O.bf16_round(-1.5) == 0xBFC0
    for b in (0x3F80, 0xC2F7, 0x0001, 0x7F7F):
        assert O.bf16_round(O.bf16_to_double(b)) == b


# ------------------------------------------------------------------ codes

def test_code_order_low_bits_first():
    words = np.full((1, 8), 0x76543210, dtype=np.uint32)
    qt = S.QTensor(words, np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16), 1, 64, 4)
    assert [O.code(qt, 0, c) for c in range(16)] == list(range(8)) * 2
    words8 = np.full((1, 16), 0x83020100, dtype=np.uint32)
    qt8 = S.QTensor(words8, np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16), 1, 64, 8)
    assert [O.code(qt8, 0, c) for c in range(8)] == [0, 1, 2, 0x83] * 2


@pytest.mark.parametrize("bits", [4, 8])
def test_codes_match_byte_view_packing(bits):
    rng = np.random.default_rng(bits)
    q = rng.integers(0, 1 << bits, size=(5, 128))
    qt = qtensor_from_codes(q, np.zeros((5, 2), np.uint16), np.zeros((5, 2), np.uint16), bits)
    assert np.array_equal(O.codes(qt), q)


@pytest.mark.parametrize("bits", [4, 8])
def test_one_hot_input_returns_dequantised_column(bits):
    rng = np.random.default_rng(10 + bits)
    rows, cols = 6, 192
    q = rng.integers(0, 1 << bits, size=(rows, cols))
    sc = f32_to_bf16_bits(rng.uniform(0.002, 0.01, (rows, cols // 64)))
    bi = f32_to_bf16_bits(rng.uniform(-1, 1, (rows, cols // 64)))
    qt = qtensor_from_codes(q, sc, bi, bits)
    s64, b64 = bf16_bits_to_f64(sc), bf16_bits_to_f64(bi)
    for c in (0, 1, 63, 64, 127, 191):
        x = np.zeros(cols)
        x[c] = 1.0
        y = O.matvec(qt, x)
        want = s64[:, c // 64] * q[:, c] + b64[:, c // 64]
        assert np.array_equal(y, want)


def test_dequant_matches_oracle_matvec_and_numpy():
    qt = S.make_qtensor(3, 0, 0, S.T_GATE_CODES, S.T_GATE_SCALES, 16, 256, 4)
    W = O.dequant(qt)
    x = np.random.default_rng(3).standard_normal(256)
    assert np.allclose(O.matvec(qt, x), W @ x, rtol=1e-13, atol=1e-13)


def test_zero_codes_closed_form():
    rng = np.random.default_rng(4)
    rows, cols = 4, 256
    bi = f32_to_bf16_bits(rng.uniform(-0.1, 0.1, (rows, cols // 64)))
    sc = f32_to_bf16_bits(rng.uniform(0.002, 0.01, (rows, cols // 64)))
    qt = qtensor_from_codes(np.zeros((rows, cols), int), sc, bi, 4)
    x = rng.standard_normal(cols)
    want = bf16_bits_to_f64(bi) @ x.reshape(cols // 64, 64).sum(axis=1)
    assert np.allclose(O.matvec(qt, x), want, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ GELU

def test_gelu_tanh_library_and_identities():
    z = np.concatenate([np.linspace(-8, 8, 401), [0.0, 1e-8, -1e-8, 30.0, -30.0]])
    want = torch.nn.functional.gelu(torch.tensor(z, dtype=torch.float64), approximate="tanh").numpy()
    got = np.array([O.gelu_tanh(v) for v in z])
    assert np.allclose(got, want, rtol=1e-14, atol=1e-15)
    assert O.gelu_tanh(0.0) == 0.0
    for v in (0.3, 1.7, 4.0):
        assert abs((O.gelu_tanh(v) - O.gelu_tanh(-v)) - v) < 1e-14


# ------------------------------------------------------------------ router

def constant_router_layer(c_bf16, H=256, E=8, k=3, router_scale=None):
    """Every router row has one constant code and one constant scale/bias."""
    layer = tiny_layer()
    rng = np.random.default_rng(5)
    qv = rng.integers(0, 256, size=E)
    sv = rng.uniform(0.002, 0.01, E)
    bv = rng.uniform(-1.0, 1.0, E)
    q = np.repeat(qv[:, None], H, axis=1)
    sc = f32_to_bf16_bits(np.repeat(sv[:, None], H // 64, axis=1))
    bi = f32_to_bf16_bits(np.repeat(bv[:, None], H // 64, axis=1))
    layer.router = qtensor_from_codes(q, sc, bi, 8)
    layer.cfg = S.LayerConfig(hidden=H, num_experts=E, inter=64, shared_inter=0, top_k=k)
    layer.router_scale = router_scale
    w_row = bf16_bits_to_f64(sc[:, 0]) * qv + bf16_bits_to_f64(bi[:, 0])
    return layer, w_row


def test_router_closed_form_constant_input():
    H = 256
    c = 0.75
    layer, w_row = constant_router_layer(c, H)
    x = f32_to_bf16_bits(np.full(H, c))
    eps = layer.cfg.eps
    # r_i = c / sqrt(c^2 + eps) / sqrt(H), so logit_e = w_e * H * r
    want = w_row * H * (c / np.sqrt(c * c + eps)) / np.sqrt(H)
    assert np.allclose(O.router_logits(layer, x), want, rtol=1e-12)


def test_router_scale_vector_closed_form():
    H = 256
    c = -1.25
    rs = np.random.default_rng(6).uniform(0.5, 2.0, H).astype(np.float32)
    layer, w_row = constant_router_layer(c, H, router_scale=rs)
    x = f32_to_bf16_bits(np.full(H, c))
    want = w_row * (c / np.sqrt(c * c + layer.cfg.eps)) / np.sqrt(H) * rs.astype(np.float64).sum()
    assert np.allclose(O.router_logits(layer, x), want, rtol=1e-12)


def test_router_rmsnorm_epsilon_placement():
    layer = tiny_layer()
    x = tiny_tokens()[0]
    xf = bf16_bits_to_f64(x)
    m = np.mean(xf * xf)
    eps = 0.5  # large epsilon makes its placement visible
    base = O.router_logits(layer, x, eps=eps)
    x2 = f32_to_bf16_bits(2.0 * xf)  # exact
    scaled = O.router_logits(layer, x2, eps=eps)
    ratio = 2.0 * np.sqrt(m + eps) / np.sqrt(4.0 * m + eps)
    assert np.allclose(scaled, base * ratio, rtol=1e-12)


def test_logit_bias_is_added():
    layer = tiny_layer()
    x = tiny_tokens()[1]
    base = O.router_logits(layer, x)
    layer.logit_bias = np.linspace(-1, 1, layer.cfg.num_experts).astype(np.float32)
    assert np.allclose(O.router_logits(layer, x) - base, layer.logit_bias.astype(np.float64), atol=1e-12)


def test_zero_input_routes_to_first_k_uniformly():
    layer = tiny_layer()
    x = np.zeros((2, layer.cfg.hidden), np.uint16)
    r = O.forward(layer, x)
    k = layer.cfg.top_k
    assert np.array_equal(r["ids"], np.tile(np.arange(k), (2, 1)))
    assert np.all(r["w"] == 1.0 / k)
    assert np.all(r["out64"] == 0.0) and np.all(r["out_bf16"] == 0)


def test_zero_input_with_zipf_bias_is_softmax_of_bias():
    cfg = S.CONFIGS["tiny"]
    layer = tiny_layer()
    layer.logit_bias = S.zipf_logit_bias(7, 0, cfg.num_experts)
    x = np.zeros((1, cfg.hidden), np.uint16)
    r = O.forward(layer, x)
    b = layer.logit_bias.astype(np.float64)
    order = np.argsort(-b, kind="stable")[: cfg.top_k]
    assert np.array_equal(r["ids"][0], order)
    assert np.allclose(r["w"][0], scipy.special.softmax(b[order]), rtol=1e-14)


def test_topk_ties_and_per_expert_scale():
    layer = tiny_layer()
    layer.cfg = S.LayerConfig(hidden=256, num_experts=6, inter=64, shared_inter=0, top_k=3)
    layer.per_expert_scale = np.array([1, 2, 3, 4, 5, 6], np.float32)
    logits = np.array([1.0, 3.0, 2.0, 3.0, -1.0, 3.0])
    ids, w = O.topk(layer, logits)
    assert list(ids) == [1, 3, 5]
    assert np.allclose(w, np.array([1, 1, 1]) / 3.0 * np.array([2, 4, 6]), rtol=1e-15)
    ids, w = O.topk(layer, np.array([0.5, -2.0, 4.0, 0.0, 0.25, 1.0]))
    assert list(ids) == [2, 5, 0]
    assert np.allclose(w, scipy.special.softmax([4.0, 1.0, 0.5]) * np.array([3, 6, 1]), rtol=1e-14)


def test_topk_selection_uses_exact_logits():
    layer = tiny_layer()
    layer.cfg = S.LayerConfig(hidden=256, num_experts=4, inter=64, shared_inter=0, top_k=1)
    # two logits that round to the same fp32 value: the exact (fp64) order decides
    ids, _ = O.topk(layer, np.array([0.0, 1.0, 1.0 + 1e-12, 0.5]))
    assert list(ids) == [2]
    ids, _ = O.topk(layer, np.array([0.0, 1.0 + 1e-12, 1.0, 0.5]))
    assert list(ids) == [1]
    # an exact tie goes to the lower index
    ids, _ = O.topk(layer, np.array([0.0, 1.0, 1.0, 0.5]))
    assert list(ids) == [1]


# ------------------------------------------------------------------ experts and layer

def test_expert_is_geglu_on_gate():
    layer = tiny_layer()
    x = bf16_bits_to_f64(tiny_tokens()[2])
    g, u, d = layer.gate.select(3), layer.up.select(3), layer.down.select(3)
    Wg, Wu, Wd = O.dequant(g), O.dequant(u), O.dequant(d)
    gt = torch.nn.functional.gelu(torch.tensor(Wg @ x), approximate="tanh").numpy()
    want = Wd @ (gt * (Wu @ x))
    assert np.allclose(O.expert(g, u, d, x), want, rtol=1e-12, atol=1e-14)


def test_dense_masked_equals_sparse_tiny():
    layer = tiny_layer()
    x = tiny_tokens()
    r = O.forward(layer, x)
    dm = O.dense_masked(layer, x)
    assert np.allclose(r["out64"], dm, rtol=1e-12, atol=1e-14)


def test_weights_sum_to_one():
    layer = tiny_layer()
    r = O.forward(layer, tiny_tokens(T=8))
    assert np.allclose(r["w"].sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(np.take_along_axis(r["logits"], r["ids"].astype(np.int64), 1), axis=1) <= 0)


def _identical_experts(layer, src=0):
    for name in ("gate", "up", "down"):
        qt = getattr(layer, name)
        for a in (qt.codes, qt.scales, qt.biases):
            a[:] = a[src]


def test_identical_experts_reduce_to_shared_plus_one():
    layer = tiny_layer()
    _identical_experts(layer)
    x = tiny_tokens()
    r = O.forward(layer, x)
    for t in range(x.shape[0]):
        xf = bf16_bits_to_f64(x[t])
        y0 = O.expert(layer.gate.select(0), layer.up.select(0), layer.down.select(0), xf)
        ys = O.expert(layer.shared_gate, layer.shared_up, layer.shared_down, xf)
        assert np.allclose(r["out64"][t], ys + y0, rtol=1e-12, atol=1e-14)
    layer.per_expert_scale = np.full(layer.cfg.num_experts, 0.25, np.float32)
    r2 = O.forward(layer, x)
    for t in range(x.shape[0]):
        xf = bf16_bits_to_f64(x[t])
        y0 = O.expert(layer.gate.select(0), layer.up.select(0), layer.down.select(0), xf)
        ys = O.expert(layer.shared_gate, layer.shared_up, layer.shared_down, xf)
        assert np.allclose(r2["out64"][t], ys + 0.25 * y0, rtol=1e-12, atol=1e-14)


def test_without_shared_expert_output_is_weighted_routed_sum():
    layer = tiny_layer()
    x = tiny_tokens()
    full = O.forward(layer, x)
    layer.shared_gate = layer.shared_up = layer.shared_down = None
    r = O.forward(layer, x)
    for t in range(x.shape[0]):
        xf = bf16_bits_to_f64(x[t])
        want = sum(r["w"][t, j] * O.expert(layer.gate.select(e), layer.up.select(e), layer.down.select(e), xf)
                   for j, e in enumerate(r["ids"][t]))
        assert np.allclose(r["out64"][t], want, rtol=1e-12, atol=1e-14)
        assert np.array_equal(full["ids"][t], r["ids"][t])


def test_expert_permutation_invariance():
    layer = tiny_layer()
    x = tiny_tokens()
    r = O.forward(layer, x)
    E = layer.cfg.num_experts
    perm = np.random.default_rng(8).permutation(E)          # new expert i = old expert perm[i]
    inv = np.argsort(perm)
    p = tiny_layer()
    for name in ("gate", "up", "down"):
        qt = getattr(p, name)
        for a in (qt.codes, qt.scales, qt.biases):
            a[:] = a[perm]
    for a in (p.router.codes, p.router.scales, p.router.biases):
        a[:] = a[perm]
    rp = O.forward(p, x)
    assert np.array_equal(rp["ids"], inv[r["ids"]])
    assert np.array_equal(rp["out64"], r["out64"])


def test_tokens_are_independent():
    layer = tiny_layer()
    x = tiny_tokens(T=6)
    r = O.forward(layer, x)
    for t in range(6):
        rt = O.forward(layer, x[t:t + 1])
        assert np.array_equal(rt["out64"][0], r["out64"][t])
        assert np.array_equal(rt["ids"][0], r["ids"][t])


def test_output_bf16_is_rounded_fp64():
    layer = tiny_layer()
    r = O.forward(layer, tiny_tokens())
    want = f32_to_bf16_bits(r["out64"].astype(np.float32))
    # fp64 -> fp32 -> bf16 can differ from a single rounding only at an exact fp32 tie
    diff = (r["out_bf16"].astype(np.int32) - want.astype(np.int32))
    assert np.count_nonzero(diff) <= 1 and np.all(np.abs(diff) <= 1)


def test_rmsnorm_bf16_closed_form_and_scale_invariance():
    H = 256
    c = 3.0
    x = f32_to_bf16_bits(np.full((1, H), c))
    y = O.rmsnorm_bf16(x, eps=1e-6)
    assert np.all(y == f32_to_bf16_bits(np.float32(c / np.sqrt(c * c + 1e-6))))
    xr = tiny_tokens(T=3)
    y1 = O.rmsnorm_bf16(xr, eps=0.0)
    y2 = O.rmsnorm_bf16(f32_to_bf16_bits(bf16_bits_to_f64(xr) * 4.0), eps=0.0)
    assert np.array_equal(y1, y2)
    yf = bf16_bits_to_f64(y1)
    assert np.allclose(np.mean(yf * yf, axis=1), 1.0, atol=2e-2)


def test_rmsnorm_bf16_epsilon_placement():
    """Constant rows with a large epsilon: y = c / sqrt(c^2 + eps) exactly
    (3 / sqrt(9 + 7) = 0.75; -1 / sqrt(1 + 3) = -0.5), so an epsilon outside
    the root or a dropped epsilon changes the value."""
    H = 128
    for c, eps, want in ((3.0, 7.0, 0.75), (-1.0, 3.0, -0.5), (0.5, 0.0, 1.0)):
        x = f32_to_bf16_bits(np.full((2, H), c))
        y = O.rmsnorm_bf16(x, eps=eps)
        assert np.all(y == f32_to_bf16_bits(np.float32(want)))
    # a mixed row: the mean of the squares sits inside the root beside eps
    xr = np.concatenate([np.full(H // 2, 2.0), np.full(H // 2, -4.0)])   # mean square 10
    y = O.rmsnorm_bf16(f32_to_bf16_bits(xr[None, :]), eps=6.0)          # sqrt(16) = 4
    assert np.array_equal(y[0], f32_to_bf16_bits(xr / 4.0))


# ------------------------------------------------------------------ group sizes and 8-bit experts

def test_group128_is_group64_with_repeated_pairs():
    """A group-128 matrix is the group-64 matrix whose adjacent groups share
    their scale and bias; one-hot inputs return column c with the pair of
    group c // 128."""
    rng = np.random.default_rng(21)
    rows, cols = 5, 256
    for bits in (4, 8):
        q = rng.integers(0, 1 << bits, size=(rows, cols))
        sc = f32_to_bf16_bits(rng.uniform(0.002, 0.01, (rows, cols // 128)))
        bi = f32_to_bf16_bits(rng.uniform(-0.1, 0.1, (rows, cols // 128)))
        q128 = qtensor_from_codes(q, sc, bi, bits)
        q128.group = 128
        q64 = qtensor_from_codes(q, np.repeat(sc, 2, axis=1), np.repeat(bi, 2, axis=1), bits)
        x = rng.standard_normal(cols)
        assert np.array_equal(O.matvec(q128, x), O.matvec(q64, x))
        s64, b64 = bf16_bits_to_f64(sc), bf16_bits_to_f64(bi)
        for c in (0, 127, 128, 200):
            e = np.zeros(cols)
            e[c] = 1.0
            assert np.array_equal(O.matvec(q128, e), s64[:, c // 128] * q[:, c] + b64[:, c // 128])


def test_dense_masked_equals_sparse_8bit_experts():
    cfg = S.LayerConfig(hidden=256, num_experts=8, inter=64, shared_inter=128, top_k=3, expert_bits=8,
                        bias_range=(-0.3, 0.3), scale_range=(1e-4, 0.02))
    layer = S.make_layer(cfg, 41)
    assert layer.gate.bits == 8 and layer.shared_down.bits == 8
    x = S.make_tokens(41, 3, cfg.hidden)
    r = O.forward(layer, x)
    assert np.allclose(r["out64"], O.dense_masked(layer, x), rtol=1e-12, atol=1e-14)
    # the expert through numpy on the dequantised matrices (independent biases)
    xf = bf16_bits_to_f64(x[1])
    e = int(r["ids"][1][0])
    g, u, d = layer.gate.select(e), layer.up.select(e), layer.down.select(e)
    h = torch.nn.functional.gelu(torch.tensor(O.dequant(g) @ xf), approximate="tanh").numpy() * (O.dequant(u) @ xf)
    assert np.allclose(O.expert(g, u, d, xf), O.dequant(d) @ h, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ layer tail

def _const_branches(H, a, b):
    return np.full(H, float(a)), np.full(H, float(b))


def test_tail_closed_form_constant_branches():
    """s = 3, r = -3 (constant rows), eps 7: each branch norm gives 3/sqrt(9 + 7)
    = 0.75 times its weight; with w_s = 1 + d and w_r = d their sum is 0.75
    everywhere, whose norm is 0.75/sqrt(0.5625 + 7) = 3/11 times w_out."""
    H = 128
    rng = np.random.default_rng(31)
    d = rng.uniform(0.1, 0.9, H).astype(np.float32)
    w_s = (1.0 + d).astype(np.float32)
    w_o = rng.uniform(0.5, 1.5, H).astype(np.float32)
    # w_s - d must be exactly 1 in fp32 for the closed form
    d = (w_s - np.float32(1.0)).astype(np.float32)
    s, r = _const_branches(H, 3.0, -3.0)
    resid = f32_to_bf16_bits(rng.standard_normal(H))
    tail = dict(norm_shared=w_s, norm_routed=d, norm_out=w_o, eps=7.0, layer_scalar=0.5)
    got = O.layer_tail(s, r, tail, resid)
    want = 0.5 * (bf16_bits_to_f64(resid) + (3.0 / 11.0) * w_o.astype(np.float64))
    assert np.allclose(got, want, rtol=1e-14, atol=1e-15)


def test_tail_without_norms_is_scaled_sum_plus_residual():
    H = 96
    rng = np.random.default_rng(32)
    s, r = rng.standard_normal(H), rng.standard_normal(H)
    resid = f32_to_bf16_bits(rng.standard_normal(H))
    got = O.layer_tail(s, r, dict(eps=1e-6, layer_scalar=1.25), resid)
    assert np.allclose(got, 1.25 * (bf16_bits_to_f64(resid) + s + r), rtol=1e-15, atol=1e-15)
    assert np.allclose(O.layer_tail(s, r, dict(eps=1e-6, layer_scalar=1.0)), s + r, rtol=0, atol=0)


def test_tail_norms_are_scale_invariant_per_branch():
    """With eps 0 each normed branch ignores its own scale."""
    H = 64
    rng = np.random.default_rng(33)
    s, r = rng.standard_normal(H), rng.standard_normal(H)
    t = S.make_tail(5, 0, H, eps=0.0)
    base = O.layer_tail(s, r, t)
    assert np.allclose(O.layer_tail(4.0 * s, 0.25 * r, t), base, rtol=1e-12, atol=1e-14)
    only_out = dict(t, norm_shared=None, norm_routed=None)
    assert np.allclose(O.layer_tail(3.0 * s, 3.0 * r, only_out), O.layer_tail(s, r, only_out), rtol=1e-12)
    assert not np.allclose(O.layer_tail(3.0 * s, r, only_out), O.layer_tail(s, r, only_out))
    # rms of the output norm's input: the output divided by its weight has unit mean square
    v = O.layer_tail(s, r, t) / t["norm_out"].astype(np.float64) / t["layer_scalar"]
    assert abs(np.mean(v * v) - 1.0) < 1e-12


def test_layer_with_tail_composes_branches():
    """The layer with a tail is the tail of (shared expert, weighted routed sum)."""
    layer = tiny_layer()
    x = tiny_tokens(T=2)
    t = S.make_tail(9, 0, layer.cfg.hidden)
    resid = tiny_tokens(seed=77, T=2)
    r = O.forward(layer, x, tail=t, resid=resid)
    base = O.forward(layer, x)
    assert np.array_equal(r["ids"], base["ids"])
    for tk in range(2):
        xf = bf16_bits_to_f64(x[tk])
        sh = O.expert(layer.shared_gate, layer.shared_up, layer.shared_down, xf)
        ro = sum(base["w"][tk, j] * O.expert(layer.gate.select(e), layer.up.select(e), layer.down.select(e), xf)
                 for j, e in enumerate(base["ids"][tk]))
        assert np.allclose(r["out64"][tk], O.layer_tail(sh, ro, t, resid[tk]), rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ quantized head

def test_head_one_hot_softcap_and_argmax():
    rng = np.random.default_rng(41)
    V, H = 40, 128
    q = rng.integers(0, 16, size=(V, H))
    sc = f32_to_bf16_bits(rng.uniform(0.2, 1.0, (V, H // 64)))
    bi = f32_to_bf16_bits(rng.uniform(-4.0, 4.0, (V, H // 64)))
    qt = qtensor_from_codes(q, sc, bi, 4)
    s64, b64 = bf16_bits_to_f64(sc), bf16_bits_to_f64(bi)
    c = 70
    x = np.zeros(H, np.uint16)
    x[c] = 0x3F80                                      # bf16 1.0
    raw = s64[:, c // 64] * q[:, c] + b64[:, c // 64]  # up to ~19: the cap matters
    lg, am = O.qgemv_head(qt, x[None, :], softcap=0.0)
    assert np.array_equal(lg[0], raw) and am[0] == int(np.argmax(raw))
    lg, am = O.qgemv_head(qt, x[None, :], softcap=5.0)
    assert np.allclose(lg[0], 5.0 * np.tanh(raw / 5.0), rtol=1e-15, atol=1e-15)
    assert np.all(np.abs(lg[0]) < 5.0) and am[0] == int(np.argmax(raw))


def test_head_argmax_ties_and_dense_rows():
    rng = np.random.default_rng(42)
    V, H = 24, 128
    q = rng.integers(0, 16, size=(V, H))
    q[17] = q[5]                                       # rows 5 and 17 identical ...
    sc = f32_to_bf16_bits(rng.uniform(0.002, 0.01, (V, H // 64)))
    sc[17] = sc[5]
    bi = f32_to_bf16_bits(rng.uniform(-0.1, 0.1, (V, H // 64)))
    bi[5] = bi[17] = f32_to_bf16_bits(np.full(H // 64, 3.0))   # ... and far above the others
    qt = qtensor_from_codes(q, sc, bi, 4)
    x = f32_to_bf16_bits(np.abs(rng.standard_normal((3, H))) + 0.1)
    lg, am = O.qgemv_head(qt, x, softcap=30.0)
    W = bf16_bits_to_f64(sc).repeat(64, axis=1) * q + bf16_bits_to_f64(bi).repeat(64, axis=1)
    raw = bf16_bits_to_f64(x) @ W.T
    assert np.allclose(lg, 30.0 * np.tanh(raw / 30.0), rtol=1e-13, atol=1e-13)
    assert np.all(am == 5)


# ------------------------------------------------------------------ the pins catch planted mistakes

def _pin_callables():
    """Every pin of this file as a no-argument callable, parametrised pins
    once per parameter value (the harness below is left out)."""
    import functools
    import inspect
    out = []
    for name, f in sorted(globals().items()):
        if not name.startswith("test_") or name == "test_planted_mistakes_are_caught" or not inspect.isfunction(f):
            continue
        params = [m for m in getattr(f, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            out.append((name, f))
            continue
        assert len(params) == 1, name
        argname, values = params[0].args
        for v in values:
            out.append(("%s[%s]" % (name, v), functools.partial(f, **{argname: v})))
    return out


# (description, exact text in moe_oracle.c, replacement)
MUTATIONS = [
    ("nibble order reversed", "(word >> (t->bits * (c % per_word)))",
     "(word >> (t->bits * (per_word - 1 - c % per_word)))"),
    ("affine bias subtracted", "(double)oq_code(t, r, c) + oq_bf16_to_double(t->biases[g])",
     "(double)oq_code(t, r, c) - oq_bf16_to_double(t->biases[g])"),
    ("scale and bias swapped", "return oq_bf16_to_double(t->scales[g]) * (double)oq_code(t, r, c) + oq_bf16_to_double(t->biases[g]);",
     "return oq_bf16_to_double(t->biases[g]) * (double)oq_code(t, r, c) + oq_bf16_to_double(t->scales[g]);"),
    ("wrong group index", "int64_t g = (int64_t)r * groups + c / gs;", "int64_t g = (int64_t)r * groups + c % groups;"),
    ("router 1/sqrt(H) dropped", "r[i] = oq_bf16_to_double(x[i]) * inv * rs * inv_sqrt_h;",
     "r[i] = oq_bf16_to_double(x[i]) * inv * rs;"),
    ("rms uses the sum", "sqrt(ss / (double)H + rt->eps)", "sqrt(ss + rt->eps)"),
    ("epsilon outside the root", "sqrt(ss / (double)H + rt->eps)", "(sqrt(ss / (double)H) + rt->eps)"),
    ("router_scale ignored", "double rs = rt->router_scale ? (double)rt->router_scale[i] : 1.0;", "double rs = 1.0;"),
    ("logit bias subtracted", "logits[e] += (double)rt->logit_bias[e];", "logits[e] -= (double)rt->logit_bias[e];"),
    ("ties to the higher index", "if (best < 0 || v > bv)", "if (best < 0 || v >= bv)"),
    ("selection picks the lowest", "if (best < 0 || v > bv)", "if (best < 0 || v < bv)"),
    ("softmax not normalised", "w[j] = exp(logits[ids[j]] - m) / den * pes;", "w[j] = exp(logits[ids[j]] - m) * pes;"),
    ("per-expert scale by slot", "(double)rt->per_expert_scale[ids[j]]", "(double)rt->per_expert_scale[j]"),
    ("GELU on the up branch", "g[i] = oq_gelu_tanh(g[i]) * u[i];", "g[i] = g[i] * oq_gelu_tanh(u[i]);"),
    ("GELU cubic coefficient", "0.044715 * z * z * z", "0.044715 * z * z"),
    ("shared expert weighted", "for (int32_t i = 0; i < H; ++i) sacc[i] = y[i];",
     "for (int32_t i = 0; i < H; ++i) sacc[i] = wt[0] * y[i];"),
    ("routed output unweighted", "racc[i] += wt[j] * y[i];", "racc[i] += y[i];"),
    ("wrong expert for the down projection", "oq_expert(&pool->gate[e], &pool->up[e], &pool->down[e], xf, y);",
     "oq_expert(&pool->gate[e], &pool->up[e], &pool->down[(e + 1) % pool->num_experts], xf, y);"),
    ("bf16 ties away from zero", "(rem == 0.5 && fmod(fl, 2.0) != 0.0)", "(rem == 0.5)"),
    ("bf16 truncates", "if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;", ""),
    ("rmsnorm without the mean", "double inv = 1.0 / sqrt(ss / (double)H + eps);", "double inv = 1.0 / sqrt(ss + eps);"),
    ("rmsnorm epsilon outside the root", "double inv = 1.0 / sqrt(ss / (double)H + eps);",
     "double inv = 1.0 / (sqrt(ss / (double)H) + eps);"),
    ("rmsnorm epsilon dropped", "double inv = 1.0 / sqrt(ss / (double)H + eps);",
     "double inv = 1.0 / sqrt(ss / (double)H);"),
    ("selection in fp32", "double v = logits[e];", "double v = (float)logits[e];"),
    ("group size ignored", "int32_t gs = t->group > 0 ? t->group : GROUP;", "int32_t gs = GROUP;"),
    ("tail epsilon outside the root", "const double inv = 1.0 / sqrt(ss / (double)H + eps);",
     "const double inv = 1.0 / (sqrt(ss / (double)H) + eps);"),
    ("tail norm weight not applied", "out[i] = v[i] * inv * (double)w[i];", "out[i] = v[i] * inv;"),
    ("tail routed norm takes the shared weight", "tail_norm(r, tail->norm_routed, H",
     "tail_norm(r, tail->norm_shared ? tail->norm_shared : tail->norm_routed, H"),
    ("tail scalar only on the FFN part", "out[i] = tail->layer_scalar * (res + b[i]);",
     "out[i] = res + tail->layer_scalar * b[i];"),
    ("tail residual dropped", "double res = resid ? oq_bf16_to_double(resid[i]) : 0.0;", "double res = 0.0;"),
    ("tail output norm skipped", "if (tail->norm_out) tail_norm(a, tail->norm_out, H, tail->eps, b);",
     "if (0) tail_norm(a, tail->norm_out, H, tail->eps, b);"),
    ("layer branches swapped into the tail", "oq_layer_tail(sacc, racc,", "oq_layer_tail(racc, sacc,"),
    ("head softcap without the inner division", "y[v] = softcap * tanh(y[v] / softcap);",
     "y[v] = softcap * tanh(y[v]);"),
    ("head argmax ties to the higher row", "if (y[v] > y[best]) best = v;", "if (y[v] >= y[best]) best = v;"),
    ("head argmax picks the lowest", "if (y[v] > y[best]) best = v;", "if (y[v] < y[best]) best = v;"),
]


@pytest.mark.slow
def test_planted_mistakes_are_caught(tmp_path):
    """Rebuild the oracle with each planted mistake and run every pin on it.
    A mistake counts as caught only when a pin fails an assertion; any other
    exception is an error of the harness or of a pin, and fails this test.
    Control: every pin first passes on the unmodified oracle, built the same
    way."""
    src = open(os.path.join(ROOT, "oracle", "moe_oracle.c")).read()
    shutil.copy(os.path.join(ROOT, "oracle", "moe_oracle.h"), tmp_path / "moe_oracle.h")
    pins = _pin_callables()
    assert len(pins) >= 25

    def first_failure():
        for name, pin in pins:
            try:
                pin()
            except AssertionError:
                return name
        return None

    ctrl = tmp_path / "control.c"
    ctrl.write_text(src)
    with O.using(O.build(force=True, src=str(ctrl), out=str(tmp_path / "control.so"))):
        assert first_failure() is None, "a pin fails on the unmodified oracle"
    missed = []
    for i, (name, old, new) in enumerate(MUTATIONS):
        assert src.count(old) >= 1, "mutation text not found: " + name
        csrc = tmp_path / ("m%d.c" % i)
        csrc.write_text(src.replace(old, new))
        lib = O.build(force=True, src=str(csrc), out=str(tmp_path / ("m%d.so" % i)))
        with O.using(lib):
            caught_by = first_failure()
        if caught_by is None:
            missed.append(name)
    assert not missed, "pins missed planted mistakes: %s" % missed

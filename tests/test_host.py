"""Host-side logic of the C-ABI library, checked without a GPU: exported
symbols, packed sizes against the pages' byte counts, the DEV_V1 layout
against its written description, the lossless pack/unpack round trip, and
argument validation (every rejected call returns before touching the GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import qmoe_synth as S
import quantized_moe_gemv_amd as M
from test_oracle_pins import page_constants

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "moegemv.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_\w+|moe_\w+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(M.EXPORTS)
    lib = ctypes.CDLL(M.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_expert_blob_sizes_match_pages():
    pc = page_constants()
    cfg = S.CONFIGS["decode"]
    H, I = cfg.hidden, cfg.inter
    blob = 2 * M.packed_bytes(I, H, 4) + M.packed_bytes(H, I, 4)
    canon = 2 * M.packed_bytes(I, H, 4, M.LAYOUT_CANONICAL) + M.packed_bytes(H, I, 4, M.LAYOUT_CANONICAL)
    assert blob == canon == 3345408        # no padding at these shapes
    pool = M.pool_layout(H, I, page_bytes=pc["page_bytes"])
    assert pool.expert_stride == pc["page_rounded_expert_blob_bytes"]
    assert pc["num_layers"] * cfg.num_experts * pool.expert_stride == pc["routed_expert_files_bytes"]
    assert pool.gate_offset == 0 and pool.up_offset == M.packed_bytes(I, H, 4)
    assert pool.down_offset == 2 * M.packed_bytes(I, H, 4)


def test_packed_bytes_rejects_unsupported():
    assert M.packed_bytes(64, 100, 4) == 0
    assert M.packed_bytes(64, 128, 3) == 0
    assert M._lib.mq_packed_bytes(64, 128, 4, 32, 1) == 0
    assert M.packed_bytes(0, 128, 4) == 0
    assert M.packed_bytes(65, 128, 4) == 2 * 2 * 2304      # rows padded to 128


def dev_word_expected(q, bits, t, g, j, lane, i):
    """The DEV_V1 word (j, lane, i) of block (t, g), from the header's description."""
    a = 4 * j + i
    if bits == 4:
        r, c0, n = 16 * (a >> 1) + lane % 16, 32 * (a & 1) + 8 * (lane // 16), 8
        pos = [4 * (e // 2) + 16 * (e % 2) for e in range(8)]
    else:
        r, c0, n = 16 * (a >> 2) + lane % 16, 16 * (a & 3) + 4 * (lane // 16), 4
        pos = [8 * e for e in range(4)]
    row = 64 * t + r
    if row >= q.shape[0]:
        return 0
    w = 0
    for e in range(n):
        w |= int(q[row, 64 * g + c0 + e]) << pos[e]
    return w


@pytest.mark.parametrize("bits,rows,cols", [(4, 64, 128), (4, 80, 192), (8, 16, 256), (8, 130, 64)])
def test_dev_layout_matches_description(bits, rows, cols):
    from test_oracle_pins import qtensor_from_codes
    rng = np.random.default_rng(rows + bits)
    q = rng.integers(0, 1 << bits, size=(rows, cols))
    sc = rng.integers(0, 1 << 16, size=(rows, cols // 64)).astype(np.uint16)
    bi = rng.integers(0, 1 << 16, size=(rows, cols // 64)).astype(np.uint16)
    qt = qtensor_from_codes(q, sc, bi, bits)
    packed = M.pack(qt)
    blk = 2304 if bits == 4 else 4352
    ncode = 2048 if bits == 4 else 4096
    G = cols // 64
    tiles = (rows + 63) // 64
    assert packed.size == tiles * G * blk
    words = packed.view("<u4")
    for t in range(tiles):
        for g in range(G):
            base = (t * G + g) * blk // 4
            for (j, lane, i) in [(0, 0, 0), (0, 17, 3), (1, 63, 1), (1, 40, 2), (bits // 4 * 2 - 1, 5, 3)]:
                got = int(words[base + (j * 64 + lane) * 4 + i])
                assert got == dev_word_expected(q, bits, t, g, j, lane, i)
            for r16 in (0, 7, 15):
                for m in range(4):
                    row = 64 * t + 16 * m + r16
                    got = int(words[base + ncode // 4 + r16 * 4 + m])
                    want = 0 if row >= rows else int(sc[row, g]) | (int(bi[row, g]) << 16)
                    assert got == want


@pytest.mark.parametrize("bits,rows,cols", [(4, 704, 2816), (4, 2816, 704), (8, 128, 2816), (4, 100, 64), (8, 16, 256)])
def test_pack_unpack_round_trip_is_exact(bits, rows, cols):
    tensor = S.T_GATE_CODES if bits == 4 else S.T_ROUTER_CODES
    qt = S.make_qtensor(11, 0, 0, tensor, tensor + 1, rows, cols, bits)
    packed = M.pack(qt)
    c, s, b = M.unpack(packed, rows, cols, bits)
    assert np.array_equal(c, qt.codes) and np.array_equal(s, qt.scales) and np.array_equal(b, qt.biases)
    if bits == 8 and rows % 64 == 0:
        # 8-bit packing moves whole bytes: the same multiset of bytes
        canon = np.concatenate([qt.codes.view(np.uint8).ravel(), qt.scales.view(np.uint8).ravel(),
                                qt.biases.view(np.uint8).ravel()])
        assert np.array_equal(np.sort(packed), np.sort(canon))


# ------------------------------------------------------------------ validation (no GPU involved)

FAKE = 1 << 32   # a 256-aligned address that is never dereferenced


def fake_layer(E=16, H=256, I=64, Is=128, k=2, bits=8):
    pool = M.pool_layout(H, I, page_bytes=4096)
    pool.base = FAKE
    pool.num_experts = E
    rw = M.MqQTensor(FAKE, None, None, E, H, bits, 64, M.LAYOUT_DEV_V1)
    router = M.MqRouter(rw, None, None, None, k, 1e-6)
    sh = M.MqShared(M.MqQTensor(FAKE, None, None, Is, H, 4, 64, 1), M.MqQTensor(FAKE, None, None, Is, H, 4, 64, 1),
                    M.MqQTensor(FAKE, None, None, H, Is, 4, 64, 1))
    return router, pool, sh


def call(router, pool, sh, T=4, H=256, ws_bytes=None, x_ptr=FAKE, out_ptr=FAKE, x_dtype=0, path=0, ws_ptr=FAKE,
         x_stride=None, in_eps=0.0):
    x = M.MqAct(x_ptr, T, H, x_dtype, H if x_stride is None else x_stride)
    out = M.MqAct(out_ptr, T, H, 0, H)
    if ws_bytes is None:
        ws_bytes = M._lib.mq_workspace_bytes(ctypes.byref(router), ctypes.byref(pool),
                                             None if sh is None else ctypes.byref(sh), max(T, 1))
    opts = M.MqOpts(path, None, None, None, ws_ptr, ws_bytes, in_eps)
    return M._lib.moe_layer_forward(ctypes.byref(x), ctypes.byref(router), ctypes.byref(pool),
                                    None if sh is None else ctypes.byref(sh), ctypes.byref(out),
                                    ctypes.byref(opts), None)


def test_zero_tokens_is_a_no_op():
    r, p, s = fake_layer()
    assert call(r, p, s, T=0, x_ptr=None, out_ptr=None, ws_ptr=None) == M.MQ_OK


def test_workspace_bytes_grows_with_tokens_and_rejects_bad_layers():
    r, p, s = fake_layer()
    f = lambda T: M._lib.mq_workspace_bytes(ctypes.byref(r), ctypes.byref(p), ctypes.byref(s), T)
    assert 0 < f(1) < f(16) < f(128)
    r.w.bits = 4
    assert f(1) == 0


@pytest.mark.parametrize("mutate,status", [
    (lambda r, p, s: setattr(r.w, "bits", 4), M.MQ_ERR_UNSUPPORTED),
    (lambda r, p, s: setattr(r.w, "group", 32), M.MQ_ERR_UNSUPPORTED),
    (lambda r, p, s: setattr(r.w, "layout", M.LAYOUT_CANONICAL), M.MQ_ERR_UNSUPPORTED),
    (lambda r, p, s: setattr(p, "bits", 6), M.MQ_ERR_UNSUPPORTED),
    (lambda r, p, s: setattr(p, "bits", 8), M.MQ_ERR_SHAPE),      # a 4-bit pool stride cannot hold 8-bit blobs
    (lambda r, p, s: setattr(p, "group", 96), M.MQ_ERR_UNSUPPORTED),
    (lambda r, p, s: setattr(p, "group", 192), M.MQ_ERR_SHAPE),   # does not divide the expert width 64
    (lambda r, p, s: setattr(s.down, "bits", 8), M.MQ_ERR_UNSUPPORTED),
    (lambda r, p, s: setattr(r, "top_k", 0), M.MQ_ERR_SHAPE),
    (lambda r, p, s: setattr(r, "top_k", 17), M.MQ_ERR_SHAPE),
    (lambda r, p, s: setattr(r.w, "rows", 15), M.MQ_ERR_SHAPE),
    (lambda r, p, s: setattr(p, "inter", 96), M.MQ_ERR_SHAPE),
    (lambda r, p, s: setattr(p, "num_experts", 300), M.MQ_ERR_SHAPE),
    (lambda r, p, s: setattr(p, "base", FAKE + 16), M.MQ_ERR_ALIGN),
    (lambda r, p, s: setattr(r.w, "codes", FAKE + 64), M.MQ_ERR_ALIGN),
    (lambda r, p, s: setattr(p, "expert_stride", p.expert_stride + 16), M.MQ_ERR_ALIGN),
    (lambda r, p, s: setattr(p, "expert_stride", 256), M.MQ_ERR_SHAPE),
    (lambda r, p, s: setattr(p, "base", None), M.MQ_ERR_NULL),
    (lambda r, p, s: setattr(s.down, "cols", 64), M.MQ_ERR_SHAPE),
    (lambda r, p, s: setattr(s.gate, "codes", None), M.MQ_ERR_NULL),
    (lambda r, p, s: setattr(s.up, "codes", FAKE + 32), M.MQ_ERR_ALIGN),
    (lambda r, p, s: setattr(r, "eps", float("nan")), M.MQ_ERR_SHAPE),
])
def test_invalid_layers_are_rejected(mutate, status):
    r, p, s = fake_layer()
    ws = M._lib.mq_workspace_bytes(ctypes.byref(r), ctypes.byref(p), ctypes.byref(s), 4)
    mutate(r, p, s)
    assert call(r, p, s, ws_bytes=ws) == status


def test_invalid_calls_are_rejected():
    r, p, s = fake_layer()
    assert call(r, p, s, ws_bytes=1000) == M.MQ_ERR_WORKSPACE
    assert call(r, p, s, ws_ptr=None) == M.MQ_ERR_WORKSPACE
    assert call(r, p, s, x_ptr=None) == M.MQ_ERR_NULL
    assert call(r, p, s, x_dtype=M.DTYPE_F32) == M.MQ_ERR_UNSUPPORTED
    assert call(r, p, s, H=128) == M.MQ_ERR_SHAPE
    assert call(r, p, s, x_ptr=FAKE + 2) == M.MQ_ERR_ALIGN
    assert call(r, p, s, x_stride=260) == M.MQ_ERR_ALIGN
    assert call(r, p, s, x_stride=100) == M.MQ_ERR_SHAPE
    assert call(r, p, s, ws_ptr=FAKE + 128) == M.MQ_ERR_ALIGN
    assert call(r, p, s, path=7) == M.MQ_ERR_UNSUPPORTED
    for bad in (-1e-6, float("nan"), float("inf")):
        assert call(r, p, s, in_eps=bad) == M.MQ_ERR_UNSUPPORTED
        assert call(r, p, s, T=0, x_ptr=None, out_ptr=None, ws_ptr=None, in_eps=bad) == M.MQ_ERR_UNSUPPORTED
    assert M._lib.moe_layer_forward(None, None, None, None, None, None, None) == M.MQ_ERR_NULL


def test_status_strings():
    for st in range(-7, 1):
        assert M.status_str(st) and M.status_str(st) != "unknown status"
    assert M.status_str(-99) == "unknown status"


def test_workspace_errors_rejects_bad_arguments():
    """Argument checks of mq_workspace_errors run before any device access."""
    v = ctypes.c_uint32(0)
    lib = M._lib
    assert lib.mq_workspace_errors(None, 4096, ctypes.byref(v), None) == M.MQ_ERR_NULL
    assert lib.mq_workspace_errors(256, 4096, None, None) == M.MQ_ERR_NULL
    assert lib.mq_workspace_errors(256 + 8, 4096, ctypes.byref(v), None) == M.MQ_ERR_ALIGN
    assert lib.mq_workspace_errors(256, 16, ctypes.byref(v), None) == M.MQ_ERR_WORKSPACE


def fake_stack(n, mutate_last=None):
    layers = [fake_layer() for _ in range(n)]
    if mutate_last:
        mutate_last(*layers[-1])
    routers = (M.MqRouter * n)(*[l[0] for l in layers])
    pools = (M.MqExpertPool * n)(*[l[1] for l in layers])
    shared = (M.MqShared * n)(*[l[2] for l in layers])
    return routers, pools, shared


def stack_call(n=3, routers=None, pools=None, shared=None, T=1, H=256, x_ptr=FAKE, out_ptr=FAKE, ws_ptr=FAKE,
               ws_bytes=None, path=0, in_eps=0.0, between_eps=0.0):
    if routers is None:
        routers, pools, shared = fake_stack(n)
    if ws_bytes is None:
        ws_bytes = M._lib.mq_stack_workspace_bytes(routers, pools, shared, n)
    x = M.MqAct(x_ptr, T, H, 0, H)
    out = M.MqAct(out_ptr, T, H, 0, H)
    opts = M.MqOpts(path, None, None, None, ws_ptr, ws_bytes, in_eps)
    return M._lib.moe_stack_forward(ctypes.byref(x), n, routers, pools, shared, between_eps, ctypes.byref(out),
                                    ctypes.byref(opts), None)


def test_stack_workspace_bytes():
    f = lambda n: M._lib.mq_stack_workspace_bytes(*fake_stack(n), n)
    assert 0 < f(1) <= f(2) < f(30)
    r, p, s = fake_layer()
    # a stack workspace also serves a one-token layer call
    assert f(1) >= M._lib.mq_workspace_bytes(ctypes.byref(r), ctypes.byref(p), ctypes.byref(s), 1)
    assert M._lib.mq_stack_workspace_bytes(*fake_stack(2), 0) == 0
    assert M._lib.mq_stack_workspace_bytes(*fake_stack(2, lambda r, p, s: setattr(p, "inter", 128)), 2) == 0
    r, p, s = fake_stack(2)
    assert M._lib.mq_stack_workspace_bytes(r, p, None, 2) > 0   # no shared expert in any layer


def test_stack_calls_are_validated_before_any_device_work():
    """Every check of moe_stack_forward that needs no device."""
    assert stack_call(n=0, ws_bytes=1 << 20) == M.MQ_ERR_SHAPE
    r, p, s = fake_stack(3, lambda r, p, s: setattr(p, "inter", 128))
    assert stack_call(3, r, p, s, ws_bytes=1 << 24) == M.MQ_ERR_SHAPE       # layers of different sizes
    r, p, s = fake_stack(3, lambda r, p, s: setattr(r.w, "bits", 4))
    assert stack_call(3, r, p, s, ws_bytes=1 << 24) == M.MQ_ERR_UNSUPPORTED
    assert stack_call(T=2) == M.MQ_ERR_SHAPE                                 # one token only
    assert stack_call(H=128) == M.MQ_ERR_SHAPE
    assert stack_call(path=M.PATHS["gemv"]) == M.MQ_ERR_UNSUPPORTED
    assert stack_call(path=M.PATHS["grouped"]) == M.MQ_ERR_UNSUPPORTED
    for bad in (-1.0, float("nan"), float("inf")):
        assert stack_call(in_eps=bad) == M.MQ_ERR_UNSUPPORTED
        assert stack_call(between_eps=bad) == M.MQ_ERR_UNSUPPORTED
    assert stack_call(x_ptr=None) == M.MQ_ERR_NULL
    assert stack_call(ws_ptr=None) == M.MQ_ERR_WORKSPACE
    assert stack_call(x_ptr=FAKE + 2) == M.MQ_ERR_ALIGN
    assert stack_call(ws_ptr=FAKE + 128) == M.MQ_ERR_ALIGN
    ws = M._lib.mq_stack_workspace_bytes(*fake_stack(3), 3)
    assert stack_call(ws_bytes=ws - 1) == M.MQ_ERR_WORKSPACE
    assert M._lib.moe_stack_forward(None, 1, None, None, None, 0.0, None, None, None) == M.MQ_ERR_NULL


# ------------------------------------------------------------------ layer tail validation (no GPU involved)

def call_with_tail(tail, T=4, H=256):
    r, p, s = fake_layer()
    x = M.MqAct(FAKE, T, H, 0, H)
    out = M.MqAct(FAKE, T, H, 0, H)
    ws_bytes = M._lib.mq_workspace_bytes(ctypes.byref(r), ctypes.byref(p), ctypes.byref(s), T)
    opts = M.MqOpts(0, None, None, None, FAKE, ws_bytes, 0.0, ctypes.addressof(tail))
    return M._lib.moe_layer_forward(ctypes.byref(x), ctypes.byref(r), ctypes.byref(p), ctypes.byref(s),
                                    ctypes.byref(out), ctypes.byref(opts), None)


def ok_tail():
    return M.MqTail(FAKE, FAKE + 1024, FAKE + 2048, FAKE + 4096, 256, 0, 1e-6, 1.0)


@pytest.mark.parametrize("field,value,status", [
    ("eps", -1.0, M.MQ_ERR_UNSUPPORTED),
    ("eps", float("nan"), M.MQ_ERR_UNSUPPORTED),
    ("layer_scalar", float("inf"), M.MQ_ERR_UNSUPPORTED),
    ("norm_shared", FAKE + 4, M.MQ_ERR_ALIGN),
    ("norm_out", FAKE + 8, M.MQ_ERR_ALIGN),
    ("residual", FAKE + 2, M.MQ_ERR_ALIGN),
    ("residual_stride", 255, M.MQ_ERR_ALIGN),
    ("residual_stride", 128, M.MQ_ERR_SHAPE),
])
def test_tail_validation(field, value, status):
    t = ok_tail()
    setattr(t, field, value)
    assert call_with_tail(t, T=0) == status          # checked before the zero-token early return


def test_tail_residual_is_input_ignores_residual_fields():
    t = ok_tail()
    t.residual_is_input = 1
    t.residual, t.residual_stride = FAKE + 2, 3
    assert call_with_tail(t, T=0) == M.MQ_OK



# ------------------------------------------------------------------ other widths of the format

@pytest.mark.parametrize("bits,group", [(4, 128), (8, 128), (4, 256), (8, 64)])
def test_pack_unpack_round_trip_other_groups(bits, group):
    rows, cols = 70, 512
    qt = S.make_qtensor(12, 0, 0, S.T_GATE_CODES, S.T_GATE_SCALES, rows, cols, bits, group=group,
                        bias_range=(-0.1, 0.1))
    assert qt.scales.shape == (rows, cols // group)
    packed = M.pack(qt)
    assert packed.size == M.packed_bytes(rows, cols, bits)     # the device layout does not depend on the group
    c, s_, b = M.unpack(packed, rows, cols, bits, group=group)
    assert np.array_equal(c, qt.codes) and np.array_equal(s_, qt.scales) and np.array_equal(b, qt.biases)
    # read back as group 64, each pair repeated over its group's blocks
    c64, s64, b64 = M.unpack(packed, rows, cols, bits, group=64)
    assert np.array_equal(s64, np.repeat(qt.scales, group // 64, axis=1))
    assert np.array_equal(b64, np.repeat(qt.biases, group // 64, axis=1))


def test_unpack_refuses_a_group_its_pairs_do_not_have():
    qt = S.make_qtensor(13, 0, 0, S.T_GATE_CODES, S.T_GATE_SCALES, 64, 256, 4)   # group 64, distinct pairs
    packed = M.pack(qt)
    with pytest.raises(M.MoeError) as e:
        M.unpack(packed, 64, 256, 4, group=128)
    assert e.value.status == M.MQ_ERR_UNSUPPORTED


def fake_layer8(E=16, H=256, I=64, Is=128, k=2):
    pool = M.pool_layout(H, I, page_bytes=4096, bits=8)
    pool.base = FAKE
    pool.num_experts = E
    router = M.MqRouter(M.MqQTensor(FAKE, None, None, E, H, 8, 64, M.LAYOUT_DEV_V1), None, None, None, k, 1e-6)
    sh = M.MqShared(M.MqQTensor(FAKE, None, None, Is, H, 8, 64, 1), M.MqQTensor(FAKE, None, None, Is, H, 8, 64, 1),
                    M.MqQTensor(FAKE, None, None, H, Is, 8, 64, 1))
    return router, pool, sh


@pytest.mark.parametrize("path,status", [(0, M.MQ_OK), (1, M.MQ_OK), (2, M.MQ_ERR_UNSUPPORTED),
                                         (3, M.MQ_ERR_UNSUPPORTED)])
def test_8bit_experts_run_on_the_gemv_kernels(path, status):
    """8-bit experts are accepted; AUTO and GEMV run them, GROUPED and FUSED
    refuse them before anything is enqueued (checked with T = 0 for the
    paths that would run, which returns before any launch)."""
    r, p, s = fake_layer8()
    T = 1 if path == 3 else 8
    got = call(r, p, s, T=T if status != M.MQ_OK else 0, path=path)
    assert got == status


# ------------------------------------------------------------------ LFU slot cache (host)

class LfuModel:
    """The slot cache written from its definition: one use per distinct
    expert per call; misses take, among the slots no expert of the call
    holds, an empty one (lowest first), else the one whose expert has the
    fewest uses, ties to the least recently used, then the lowest slot."""

    def __init__(self, E, S):
        self.E, self.S = E, S
        self.slot_of, self.expert_of = {}, [-1] * S
        self.uses, self.last, self.clock = [0] * E, [0] * S, 0

    def plan(self, ids):
        distinct = list(dict.fromkeys(int(e) for e in ids))
        if len(distinct) > self.S or any(not 0 <= e < self.E for e in distinct):
            raise ValueError
        self.clock += 1
        held = {self.slot_of[e] for e in distinct if e in self.slot_of}
        for e in distinct:
            self.uses[e] += 1
        fills = []
        for e in distinct:
            if e in self.slot_of:
                continue
            free = [s for s in range(self.S) if s not in held]
            empty = [s for s in free if self.expert_of[s] < 0]
            s = min(empty) if empty else min(free, key=lambda q: (self.uses[self.expert_of[q]], self.last[q], q))
            if self.expert_of[s] >= 0:
                del self.slot_of[self.expert_of[s]]
            self.expert_of[s], self.slot_of[e] = e, s
            held.add(s)
            fills.append((e, s))
        for e in distinct:
            self.last[self.slot_of[e]] = self.clock
        return [self.slot_of[int(e)] for e in ids], fills


def test_lfu_matches_its_definition_over_a_long_skewed_sequence():
    rng = np.random.default_rng(3)
    E, S = 40, 7
    p = np.arange(1, E + 1, dtype=float) ** -1.1
    p /= p.sum()
    c, m = M.LfuCache(E, S), LfuModel(E, S)
    hits = 0
    for call in range(600):
        n = int(rng.integers(1, 9))
        ids = rng.choice(E, size=n, p=p)
        while len(set(ids.tolist())) > S:
            ids = ids[:-1]
        got_slots, got_fills = c.plan(ids)
        want_slots, want_fills = m.plan(ids)
        assert got_slots.tolist() == want_slots and got_fills == want_fills, call
        hits += len(set(ids.tolist())) - len(got_fills)
    assert 0 < hits < 600 * 8


def test_lfu_never_two_fills_into_one_slot_and_keeps_the_calls_experts():
    c = M.LfuCache(16, 4)
    slots, fills = c.plan(np.array([3, 5, 3, 7]))
    assert sorted(s for _, s in fills) == [0, 1, 2] and slots.tolist()[0] == slots.tolist()[2]
    slots, fills = c.plan(np.array([9, 3, 11]))      # 3 stays; 9 and 11 need two slots, one of them empty
    assert len({s for _, s in fills}) == 2 and slots[1] == 0 and 3 not in [e for e, _ in fills]


def test_lfu_refuses_more_experts_than_slots_and_bad_ids_without_changing_state():
    c2 = M.LfuCache(16, 3)
    m2 = LfuModel(16, 3)
    c2.plan(np.array([1, 2]))
    m2.plan([1, 2])
    for bad in ([1, 2, 3, 4], [0, 16], [-1]):
        with pytest.raises(M.MoeError) as e:
            c2.plan(np.array(bad))
        assert e.value.status == M.MQ_ERR_SHAPE
    s, f = c2.plan(np.array([5, 1]))
    ws, wf = m2.plan([5, 1])
    assert s.tolist() == ws and f == wf

"""Seeded synthetic inputs for the quantized MoE FFN layer.

Test and benchmark infrastructure shared by the CPU oracle and the GPU path.
It draws random codes, bf16 scales/biases, bf16 activations and the Zipf
logit skew, and holds none of the layer's arithmetic.  Every tensor comes
out in the canonical MLX-affine layout: for a [rows][cols] matrix with b-bit
codes, ``codes`` is uint32 [rows][cols*b/32] (element c of a row in word
c/(32/b) at bit b*(c % (32/b)), low bits first), ``scales`` and ``biases``
are bf16 bit patterns (uint16) [rows][cols/64].

Recipe (all draws from the counter-based SplitMix64 streams in synth.c,
keyed by (seed, layer, expert, tensor)):
  * codes: uniform random 32-bit words, i.e. i.i.d. uniform codes;
  * scale: bf16(U[0.002, 0.01]); bias: -2^(b-1) * scale (exact in bf16);
    or, for the general affine map, scale and bias drawn independently
    (bf16 of uniforms over given ranges, from streams of their own);
  * group: 64 weights per scale/bias (other sizes on request);
  * activations: bf16(N(0, 1)) by Box-Muller;
  * Zipf skew (128-token and 4096-token prefill): an additive per-expert
    logit bias 0.37 * ln p_pi(e), p_k = k^-1.1 / sum_j j^-1.1, pi a seeded
    permutation of the experts.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqmoe_synth.so")
_lib = None
_lib_lock = threading.Lock()

GROUP = 64

# tensor ids inside a stream key
T_ROUTER_CODES, T_ROUTER_SCALES = 1, 2
T_GATE_CODES, T_GATE_SCALES = 3, 4
T_UP_CODES, T_UP_SCALES = 5, 6
T_DOWN_CODES, T_DOWN_SCALES = 7, 8
T_SGATE_CODES, T_SGATE_SCALES = 9, 10
T_SUP_CODES, T_SUP_SCALES = 11, 12
T_SDOWN_CODES, T_SDOWN_SCALES = 13, 14
T_TOKENS = 15
T_ZIPF_PERM = 16
T_BIAS_FLAG = 0x100     # or-ed into a scale stream id: the independent-bias stream
T_TAIL = 17             # layer-tail norm weights
SHARED_SLOT = 0xFFFF


def build(force: bool = False) -> str:
    """Compile synth.c into libqmoe_synth.so with gcc."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            u64, ptr, f32 = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_float
            lib.synth_u32.argtypes = [u64, u64, u64, u64, ptr]
            lib.synth_u64.argtypes = [u64, u64, u64, u64, ptr]
            lib.synth_uniform_bf16.argtypes = [u64, u64, u64, u64, f32, f32, ptr]
            lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, ptr]
            lib.synth_neg_mul_bf16.argtypes = [ptr, u64, f32, ptr]
            for f in (lib.synth_u32, lib.synth_u64, lib.synth_uniform_bf16,
                      lib.synth_normal_bf16, lib.synth_neg_mul_bf16):
                f.restype = None
            _lib = lib
    return _lib


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))
    return _POOL


def stream_id(layer: int, slot: int, tensor: int) -> int:
    return ((layer & 0xFFFF) << 32) | ((slot & 0xFFFF) << 16) | (tensor & 0xFFFF)


_TLS = threading.local()


def _chunked(fn, n: int, chunk: int = 1 << 22):
    # Inside a pool worker run inline: waiting on the pool from a worker could deadlock.
    if n <= chunk or getattr(_TLS, "in_pool", False):
        fn(0, n)
        return
    futs = [_pool().submit(fn, s, min(chunk, n - s)) for s in range(0, n, chunk)]
    for f in futs:
        f.result()


def rand_u32(seed: int, stream: int, n: int) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.uint32)
    base = out.ctypes.data

    def fn(s, c):
        lib.synth_u32(seed, stream, s, c, base + 4 * s)
    _chunked(fn, n)
    return out


def rand_u64(seed: int, stream: int, n: int) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.uint64)
    lib.synth_u64(seed, stream, 0, n, out.ctypes.data)
    return out


def uniform_bf16(seed: int, stream: int, n: int, lo: float, hi: float) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.uint16)
    base = out.ctypes.data

    def fn(s, c):
        lib.synth_uniform_bf16(seed, stream, s, c, lo, hi, base + 2 * s)
    _chunked(fn, n)
    return out


def normal_bf16(seed: int, stream: int, n: int) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.uint16)
    base = out.ctypes.data

    def fn(s, c):
        lib.synth_normal_bf16(seed, stream, s, c, base + 2 * s)
    _chunked(fn, n)
    return out


def neg_mul_bf16(scales: np.ndarray, mid: float) -> np.ndarray:
    lib = _load()
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.empty_like(s)
    lib.synth_neg_mul_bf16(s.ctypes.data, s.size, mid, out.ctypes.data)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class QTensor:
    """A group-64 MLX-affine quantized matrix in canonical layout (host arrays).

    ``codes`` may carry leading batch dimensions (e.g. [E][rows][words]) when
    several matrices of one shape are stored together.
    """
    codes: np.ndarray      # uint32 [..., rows, cols*bits/32]
    scales: np.ndarray     # uint16 (bf16 bits) [..., rows, cols/64]
    biases: np.ndarray     # uint16 (bf16 bits) [..., rows, cols/64]
    rows: int
    cols: int
    bits: int
    group: int = GROUP

    def select(self, i: int) -> "QTensor":
        return QTensor(self.codes[i], self.scales[i], self.biases[i], self.rows, self.cols, self.bits, self.group)


def make_qtensor(seed: int, layer: int, slot: int, t_codes: int, t_scales: int,
                 rows: int, cols: int, bits: int, batch: int = 0,
                 scale_lo: float = 0.002, scale_hi: float = 0.01,
                 bias_range: Optional[tuple] = None, group: int = GROUP) -> QTensor:
    """Uniform random codes, bf16 scale ~ U[scale_lo, scale_hi], and
    bias = -2^(bits-1)*scale, or with ``bias_range`` = (lo, hi) a bias
    bf16(U[lo, hi]) drawn independently of the scale.  One scale and bias per
    ``group`` weights of a row.

    With ``batch`` > 0 the result holds ``batch`` matrices, matrix i drawn from
    the streams of slot ``slot + i`` (one expert per slot).
    """
    assert cols % group == 0 and 32 % bits == 0
    words = cols * bits // 32
    groups = cols // group
    nb = max(batch, 1)
    codes = np.empty((nb, rows, words), dtype=np.uint32)
    scales = np.empty((nb, rows, groups), dtype=np.uint16)

    def one(i):
        _TLS.in_pool = nb > 1
        codes[i] = rand_u32(seed, stream_id(layer, slot + i, t_codes), rows * words).reshape(rows, words)
        scales[i] = uniform_bf16(seed, stream_id(layer, slot + i, t_scales), rows * groups,
                                 scale_lo, scale_hi).reshape(rows, groups)
    if nb > 1:
        list(_pool().map(one, range(nb)))
    else:
        one(0)
    if bias_range is None:
        biases = neg_mul_bf16(scales, float(1 << (bits - 1)))
    else:
        biases = np.stack([uniform_bf16(seed, stream_id(layer, slot + i, t_scales | T_BIAS_FLAG), rows * groups,
                                        bias_range[0], bias_range[1]).reshape(rows, groups) for i in range(nb)])
    if batch == 0:
        codes, scales, biases = codes[0], scales[0], biases[0]
    return QTensor(codes, scales, biases, rows, cols, bits, group)


def zipf_logit_bias(seed: int, layer: int, num_experts: int, s: float = 1.1,
                    strength: float = 0.37) -> np.ndarray:
    """Per-expert additive logit bias strength * ln p_pi(e), Zipf(s) over a seeded permutation."""
    k = np.arange(1, num_experts + 1, dtype=np.float64)
    p = k ** (-s)
    p /= p.sum()
    draws = rand_u64(seed, stream_id(layer, SHARED_SLOT, T_ZIPF_PERM), num_experts)
    perm = np.arange(num_experts)
    for i in range(num_experts - 1, 0, -1):         # Fisher-Yates
        j = int(draws[i] % np.uint64(i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return (strength * np.log(p[perm])).astype(np.float32)


@dataclass
class LayerConfig:
    hidden: int
    num_experts: int
    inter: int
    shared_inter: int
    top_k: int
    tokens: int = 1
    zipf: bool = False
    eps: float = 1e-6
    name: str = ""
    expert_bits: int = 4            # routed and shared expert codes (4 or 8)
    group: int = GROUP              # weights per scale/bias of the expert matrices
    scale_range: tuple = (0.002, 0.01)
    bias_range: Optional[tuple] = None   # None: bias = -2^(b-1) * scale


# The five synthetic workloads (Gemma-4-26B-A4B shapes except the first).
CONFIGS = {
    "tiny": LayerConfig(hidden=256, num_experts=16, inter=64, shared_inter=128, top_k=2,
                        tokens=4, name="tiny 4-token layer (H256 E16 I64 Is128 k2)"),
    "decode": LayerConfig(hidden=2816, num_experts=128, inter=704, shared_inter=2112, top_k=8,
                          tokens=1, name="Gemma-4-26B-A4B MoE layer, 1-token decode"),
    "prefill128": LayerConfig(hidden=2816, num_experts=128, inter=704, shared_inter=2112, top_k=8,
                              tokens=128, zipf=True,
                              name="Gemma-4-26B-A4B MoE layer, 128-token prefill, Zipf(1.1) routing"),
    "stack30": LayerConfig(hidden=2816, num_experts=128, inter=704, shared_inter=2112, top_k=8,
                           tokens=1, name="30-layer decode stack of Gemma-4-26B-A4B MoE layers"),
    "prefill4096": LayerConfig(hidden=2816, num_experts=128, inter=704, shared_inter=2112, top_k=8,
                               tokens=4096, zipf=True,
                               name="Gemma-4-26B-A4B MoE layer, 4096-token prefill, Zipf(1.1) routing"),
}
SEEDS = {"tiny": 0x5EED0000, "decode": 0x5EED0001, "prefill128": 0x5EED0002,
         "stack30": 0x5EED0003, "prefill4096": 0x5EED0004}


@dataclass
class Layer:
    """One synthetic MoE FFN layer in canonical layout (host memory)."""
    cfg: LayerConfig
    router: QTensor                     # [E][H], 8-bit
    gate: QTensor                       # [E][I][H], 4-bit
    up: QTensor                         # [E][I][H], 4-bit
    down: QTensor                       # [E][H][I], 4-bit
    shared_gate: Optional[QTensor]      # [Is][H]
    shared_up: Optional[QTensor]        # [Is][H]
    shared_down: Optional[QTensor]      # [H][Is]
    router_scale: Optional[np.ndarray] = None     # float32 [H]
    per_expert_scale: Optional[np.ndarray] = None  # float32 [E]
    logit_bias: Optional[np.ndarray] = None        # float32 [E]
    seed: int = 0
    index: int = 0


def _qkw(cfg: LayerConfig) -> dict:
    return dict(scale_lo=cfg.scale_range[0], scale_hi=cfg.scale_range[1], bias_range=cfg.bias_range,
                group=cfg.group)


def make_expert(cfg: LayerConfig, seed: int, layer: int, expert: int):
    """(gate, up, down) of one routed expert; the same values make_layer draws for it."""
    H, I, b, kw = cfg.hidden, cfg.inter, cfg.expert_bits, _qkw(cfg)
    return (make_qtensor(seed, layer, expert, T_GATE_CODES, T_GATE_SCALES, I, H, b, **kw),
            make_qtensor(seed, layer, expert, T_UP_CODES, T_UP_SCALES, I, H, b, **kw),
            make_qtensor(seed, layer, expert, T_DOWN_CODES, T_DOWN_SCALES, H, I, b, **kw))


def make_layer(cfg: LayerConfig, seed: int, layer: int = 0, shared: bool = True, experts: bool = True) -> Layer:
    """A full layer; with experts=False the routed experts are left out (None)."""
    H, E, I, Is = cfg.hidden, cfg.num_experts, cfg.inter, cfg.shared_inter
    b, kw = cfg.expert_bits, _qkw(cfg)
    router = make_qtensor(seed, layer, SHARED_SLOT, T_ROUTER_CODES, T_ROUTER_SCALES, E, H, 8)
    gate = up = down = None
    if experts:
        gate = make_qtensor(seed, layer, 0, T_GATE_CODES, T_GATE_SCALES, I, H, b, batch=E, **kw)
        up = make_qtensor(seed, layer, 0, T_UP_CODES, T_UP_SCALES, I, H, b, batch=E, **kw)
        down = make_qtensor(seed, layer, 0, T_DOWN_CODES, T_DOWN_SCALES, H, I, b, batch=E, **kw)
    sg = su = sd = None
    if shared and Is > 0:
        sg = make_qtensor(seed, layer, SHARED_SLOT, T_SGATE_CODES, T_SGATE_SCALES, Is, H, b, **kw)
        su = make_qtensor(seed, layer, SHARED_SLOT, T_SUP_CODES, T_SUP_SCALES, Is, H, b, **kw)
        sd = make_qtensor(seed, layer, SHARED_SLOT, T_SDOWN_CODES, T_SDOWN_SCALES, H, Is, b, **kw)
    bias = zipf_logit_bias(seed, layer, E) if cfg.zipf else None
    return Layer(cfg, router, gate, up, down, sg, su, sd, None, None, bias, seed, layer)


def make_tokens(seed: int, T: int, H: int, batch: int = 0, layer: int = 0) -> np.ndarray:
    """bf16 bit patterns [T][H] of N(0, 1) activations."""
    return normal_bf16(seed, stream_id(layer, batch, T_TOKENS), T * H).reshape(T, H)


def make_tail(seed: int, layer: int, H: int, norms=("shared", "routed", "out"), layer_scalar: float = 0.75,
              eps: float = 1e-6) -> dict:
    """Layer-tail parameters: learned post-FFN norm weights U[0.5, 1.5] (fp32,
    rounded through bf16 as a checkpoint stores them) for the named norms, the
    layer scalar and epsilon."""
    out = dict(eps=eps, layer_scalar=layer_scalar)
    for i, n in enumerate(("shared", "routed", "out")):
        w = None
        if n in norms:
            w = bf16_bits_to_f32(uniform_bf16(seed, stream_id(layer, SHARED_SLOT, T_TAIL) + (i << 20), H, 0.5, 1.5))
        out["norm_" + n] = w
    return out


# Vocabulary of the synthetic tied head: the pages do not give it; 262,144
# rows (2^18) stands in for the Gemma tokenizer's vocabulary.
HEAD_VOCAB = 262144
T_HEAD_CODES, T_HEAD_SCALES = 18, 19


def make_head(seed: int, vocab: int, H: int, bits: int = 4) -> QTensor:
    """The tied embedding/head matrix [vocab][H], drawn like the expert matrices."""
    return make_qtensor(seed, 0, SHARED_SLOT, T_HEAD_CODES, T_HEAD_SCALES, vocab, H, bits)

"""Python binding of libmoegemv (the MI355X quantized MoE FFN layer).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI of ``include/moegemv.h``.  PyTorch provides device memory
and the stream; the library never allocates.  Importing this package fails
with an ImportError when the HIP library has not been built (run
``python quantized_moe_gemv_amd/build.py``); there is no CPU fallback.
"""
from __future__ import annotations

import copy
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
import torch  # loads the HIP runtime that libmoegemv then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoegemv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libmoegemv.so is not built: run `python quantized_moe_gemv_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

MQ_OK, MQ_ERR_NULL, MQ_ERR_SHAPE, MQ_ERR_ALIGN = 0, -1, -2, -3
MQ_ERR_UNSUPPORTED, MQ_ERR_WORKSPACE, MQ_ERR_HIP, MQ_ERR_BUFFER = -4, -5, -6, -7
MQ_ERR_TOO_LARGE = -8
LAYOUT_CANONICAL, LAYOUT_DEV_V1 = 0, 1
DTYPE_BF16, DTYPE_F32 = 0, 1
PATHS = {"auto": 0, "gemv": 1, "grouped": 2, "fused": 3}
GROUP = 64
EXPORTS = ["moe_layer_forward", "mq_workspace_bytes", "moe_stack_forward", "mq_stack_workspace_bytes", "mq_workspace_errors", "mq_rmsnorm", "mq_packed_bytes", "mq_pool_layout",
           "mq_pack", "mq_unpack", "mq_debug_unpack_codes", "mq_debug_dequant", "mq_stream_read",
           "moe_layer_forward_noalloc", "mq_noalloc_scratch_bytes", "mq_qgemv", "mq_qgemv_workspace_bytes",
           "mq_route", "mq_route_workspace_bytes", "mq_lfu_state_bytes", "mq_lfu_init", "mq_lfu_plan",
           "mq_status_str"]


class MqQTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("layout", ctypes.c_int32)]


class MqRouter(ctypes.Structure):
    _fields_ = [("w", MqQTensor), ("router_scale", ctypes.c_void_p), ("per_expert_scale", ctypes.c_void_p),
                ("logit_bias", ctypes.c_void_p), ("top_k", ctypes.c_int32), ("eps", ctypes.c_float)]


class MqExpertPool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("expert_stride", ctypes.c_int64), ("gate_offset", ctypes.c_int64),
                ("up_offset", ctypes.c_int64), ("down_offset", ctypes.c_int64),
                ("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("layout", ctypes.c_int32)]


class MqShared(ctypes.Structure):
    _fields_ = [("gate", MqQTensor), ("up", MqQTensor), ("down", MqQTensor)]


class MqAct(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("row_stride", ctypes.c_int64)]


class MqTail(ctypes.Structure):
    _fields_ = [("norm_shared", ctypes.c_void_p), ("norm_routed", ctypes.c_void_p), ("norm_out", ctypes.c_void_p),
                ("residual", ctypes.c_void_p), ("residual_stride", ctypes.c_int64),
                ("residual_is_input", ctypes.c_int32), ("eps", ctypes.c_float), ("layer_scalar", ctypes.c_float)]


class MqOpts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("input_rmsnorm_eps", ctypes.c_float), ("tail", ctypes.c_void_p),
                ("route_ids", ctypes.c_void_p), ("route_w", ctypes.c_void_p), ("route_slots", ctypes.c_void_p),
                ("experts_ready", ctypes.c_void_p)]


class Tail:
    """Layer-tail parameters on the device: post-FFN norm weights (fp32 [H] or
    None), a residual (bf16 [T][H] tensor, None, or residual_is_input), the
    epsilon and the layer scalar."""

    def __init__(self, norm_shared=None, norm_routed=None, norm_out=None, residual: Optional[torch.Tensor] = None,
                 residual_is_input: bool = False, eps: float = 1e-6, layer_scalar: float = 1.0, device="cuda"):
        dev = lambda a: None if a is None else torch.as_tensor(np.asarray(a, np.float32)).to(device)
        self.w = [dev(norm_shared), dev(norm_routed), dev(norm_out)]
        self.residual = residual
        ptr = lambda t: None if t is None else t.data_ptr()
        self.struct = MqTail(ptr(self.w[0]), ptr(self.w[1]), ptr(self.w[2]), ptr(residual),
                             0 if residual is None else residual.stride(0), int(bool(residual_is_input)),
                             float(eps), float(layer_scalar))

    @classmethod
    def from_dict(cls, d: dict, **kw) -> "Tail":
        return cls(d.get("norm_shared"), d.get("norm_routed"), d.get("norm_out"), eps=d.get("eps", 1e-6),
                   layer_scalar=d.get("layer_scalar", 1.0), **kw)


_P = ctypes.c_void_p
_sig = {
    "mq_workspace_bytes": (ctypes.c_size_t, [_P, _P, _P, ctypes.c_int32]),
    "moe_layer_forward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "mq_stack_workspace_bytes": (ctypes.c_size_t, [_P, _P, _P, ctypes.c_int32]),
    "moe_stack_forward": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, _P, ctypes.c_float, _P, _P, _P]),
    "mq_rmsnorm": (ctypes.c_int, [_P, _P, ctypes.c_float, _P]),
    "mq_workspace_errors": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
    "mq_packed_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 5),
    "mq_pool_layout": (ctypes.c_int64, [ctypes.c_int32] * 4 + [ctypes.c_int64, _P]),
    "mq_pack": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "mq_unpack": (ctypes.c_int, [_P, _P, _P, _P]),
    "mq_debug_unpack_codes": (ctypes.c_int, [_P, _P, _P]),
    "mq_debug_dequant": (ctypes.c_int, [_P, _P, _P]),
    "mq_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, ctypes.c_int32, _P]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "mq_qgemv_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "mq_route_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32]),
    "mq_route": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "mq_lfu_state_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "mq_lfu_init": (ctypes.c_int, [_P, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32]),
    "mq_lfu_plan": (ctypes.c_int, [_P, ctypes.c_size_t, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "mq_qgemv": (ctypes.c_int, [_P, _P, _P, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]),
    "mq_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "mq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s (status %d)" % (what, status_str(status), status))
        self.status = status


def status_str(s: int) -> str:
    return _lib.mq_status_str(s).decode()


def _check(status: int, what: str):
    if status != MQ_OK:
        raise MoeError(status, what)


def _ref(s) -> Optional[ctypes._Pointer]:
    return None if s is None else ctypes.byref(s)


def _stream_handle(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ------------------------------------------------------------------ host packing

def packed_bytes(rows: int, cols: int, bits: int, layout: int = LAYOUT_DEV_V1, group: int = GROUP) -> int:
    return int(_lib.mq_packed_bytes(rows, cols, bits, group, layout))


def _canonical_desc(qt) -> tuple:
    c = np.ascontiguousarray(qt.codes, dtype=np.uint32)
    s = np.ascontiguousarray(qt.scales, dtype=np.uint16)
    b = np.ascontiguousarray(qt.biases, dtype=np.uint16)
    d = MqQTensor(c.ctypes.data, s.ctypes.data, b.ctypes.data, qt.rows, qt.cols, qt.bits, _group(qt),
                  LAYOUT_CANONICAL)
    return d, (c, s, b)


def _group(qt) -> int:
    return int(getattr(qt, "group", GROUP))


def pack_into(qt, dst: np.ndarray, offset: int = 0) -> int:
    """Pack a canonical host tensor into dst[offset:] (uint8); returns the byte count."""
    n = packed_bytes(qt.rows, qt.cols, qt.bits, group=_group(qt))
    assert dst.dtype == np.uint8 and dst.flags.c_contiguous and offset + n <= dst.size
    d, keep = _canonical_desc(qt)
    _check(_lib.mq_pack(ctypes.byref(d), dst.ctypes.data + offset, n, None), "mq_pack")
    return n


def pack(qt) -> np.ndarray:
    out = np.empty(packed_bytes(qt.rows, qt.cols, qt.bits, group=_group(qt)), dtype=np.uint8)
    pack_into(qt, out)
    return out


def unpack(packed: np.ndarray, rows: int, cols: int, bits: int, group: int = GROUP):
    """DEV_V1 host bytes -> canonical (codes uint32, scales uint16, biases uint16)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    codes = np.empty((rows, cols * bits // 32), np.uint32)
    scales = np.empty((rows, cols // group), np.uint16)
    biases = np.empty((rows, cols // group), np.uint16)
    d = MqQTensor(packed.ctypes.data, None, None, rows, cols, bits, group, LAYOUT_DEV_V1)
    _check(_lib.mq_unpack(ctypes.byref(d), codes.ctypes.data, scales.ctypes.data, biases.ctypes.data), "mq_unpack")
    return codes, scales, biases


def pool_layout(hidden: int, inter: int, page_bytes: int = 16384, bits: int = 4, group: int = GROUP) -> MqExpertPool:
    pool = MqExpertPool()
    stride = _lib.mq_pool_layout(hidden, inter, bits, group, page_bytes, ctypes.byref(pool))
    if stride <= 0:
        raise MoeError(MQ_ERR_SHAPE, "mq_pool_layout")
    return pool


def pack_expert_into(pool: MqExpertPool, e: int, gate, up, down, host: np.ndarray) -> None:
    """Pack one expert's canonical (gate, up, down) into its blob of a host pool buffer."""
    base = e * pool.expert_stride
    pack_into(gate, host, base + pool.gate_offset)
    pack_into(up, host, base + pool.up_offset)
    pack_into(down, host, base + pool.down_offset)


# ------------------------------------------------------------------ device layer

class DeviceLayer:
    """A layer packed to DEV_V1 and resident in device memory (torch tensors).

    ``src`` is a canonical host layer (``qmoe_synth.Layer`` or anything with
    the same fields).  The routed experts live in one buffer of
    num_experts * expert_stride bytes, each blob page-rounded.
    """

    def __init__(self, src, device="cuda", page_bytes: int = 16384, threads: int = 16,
                 pool_host: Optional[np.ndarray] = None, resident_experts: bool = True):
        cfg = src.cfg
        self.hidden, self.num_experts, self.inter = cfg.hidden, cfg.num_experts, cfg.inter
        self.top_k, self.eps = cfg.top_k, cfg.eps
        self.shared_inter = 0 if src.shared_gate is None else src.shared_gate.rows
        E = self.num_experts
        self.pool = pool_layout(self.hidden, self.inter, page_bytes, bits=src.gate.bits if src.gate is not None
                                else getattr(cfg, "expert_bits", 4), group=_group(src.gate) if src.gate is not None
                                else getattr(cfg, "group", GROUP))
        stride = self.pool.expert_stride
        if not resident_experts:
            # the experts live elsewhere (OffloadedLayer): no device pool here
            self.pool_buf = None
            self.pool.num_experts = E
            host = None
        elif pool_host is not None:
            # experts already packed by the caller (e.g. with pack_pool_into)
            assert pool_host.dtype == np.uint8 and pool_host.size == E * stride
            host = pool_host
        else:
            host = np.zeros(E * stride, dtype=np.uint8)

            def pack_expert(e):
                pack_expert_into(self.pool, e, src.gate.select(e), src.up.select(e), src.down.select(e), host)
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(pack_expert, range(E)))
        if host is not None:
            self.pool_buf = torch.from_numpy(host).to(device)
            del host
            self.pool.base = self.pool_buf.data_ptr()
            self.pool.num_experts = E

        def dev_tensor(qt):
            buf = torch.from_numpy(pack(qt)).to(device)
            return buf, MqQTensor(buf.data_ptr(), None, None, qt.rows, qt.cols, qt.bits, _group(qt), LAYOUT_DEV_V1)

        self.router_buf, self.router_w = dev_tensor(src.router)
        opt = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
        self.router_scale = opt(src.router_scale)
        self.per_expert_scale = opt(src.per_expert_scale)
        self.logit_bias = opt(src.logit_bias)
        ptr = lambda t: None if t is None else t.data_ptr()
        self.router = MqRouter(self.router_w, ptr(self.router_scale), ptr(self.per_expert_scale),
                               ptr(self.logit_bias), self.top_k, self.eps)
        self.shared = None
        if src.shared_gate is not None:
            self.sg_buf, sg = dev_tensor(src.shared_gate)
            self.su_buf, su = dev_tensor(src.shared_up)
            self.sd_buf, sd = dev_tensor(src.shared_down)
            self.shared = MqShared(sg, su, sd)

    def with_logit_bias(self, bias: Optional[torch.Tensor]) -> "DeviceLayer":
        """The same resident layer with another additive router score bias."""
        other = copy.copy(self)
        other.logit_bias = bias
        other.router = MqRouter(self.router_w, self.router.router_scale, self.router.per_expert_scale,
                                None if bias is None else bias.data_ptr(), self.top_k, self.eps)
        return other

    def workspace_bytes(self, max_tokens: int) -> int:
        n = _lib.mq_workspace_bytes(ctypes.byref(self.router), ctypes.byref(self.pool), _ref(self.shared),
                                    max_tokens)
        if n == 0:
            raise MoeError(MQ_ERR_SHAPE, "mq_workspace_bytes")
        return int(n)

    def new_workspace(self, max_tokens: int, device="cuda") -> torch.Tensor:
        return torch.zeros(self.workspace_bytes(max_tokens), dtype=torch.uint8, device=device)

    def weight_bytes(self) -> int:
        n = self.router_buf.numel() + (0 if self.pool_buf is None else self.pool_buf.numel())
        if self.shared is not None:
            n += self.sg_buf.numel() + self.su_buf.numel() + self.sd_buf.numel()
        return n


def _act(t: torch.Tensor) -> MqAct:
    assert t.dim() == 2 and t.stride(1) == 1
    dt = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}[t.dtype]
    return MqAct(t.data_ptr(), t.shape[0], t.shape[1], dt, t.stride(0))


def moe_layer_forward(layer: DeviceLayer, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, path: str = "auto",
                      out_dtype=torch.bfloat16, topk_ids: Optional[torch.Tensor] = None,
                      topk_w: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                      stream=None, input_rmsnorm_eps: float = 0.0, tail: Optional[Tail] = None,
                      route_ids: Optional[torch.Tensor] = None, route_w: Optional[torch.Tensor] = None,
                      route_slots: Optional[torch.Tensor] = None, experts_ready=None) -> torch.Tensor:
    """out = shared(x) + sum_j w_j expert_j(x) on the current (or given) stream.
    input_rmsnorm_eps > 0 applies a unit-weight RMSNorm (rounded to bf16) to x first;
    ``tail`` applies the layer tail (post-FFN norms, residual, layer scalar)."""
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, layer.hidden), dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = layer.new_workspace(T, x.device)
    xa, oa = _act(x), _act(out)
    ptr = lambda t: None if t is None else t.data_ptr()
    opts = MqOpts(PATHS[path], ptr(topk_ids), ptr(topk_w), ptr(logits), workspace.data_ptr(), workspace.numel(),
                  float(input_rmsnorm_eps), None if tail is None else ctypes.addressof(tail.struct),
                  ptr(route_ids), ptr(route_w), ptr(route_slots),
                  None if experts_ready is None else experts_ready.cuda_event)
    st = _lib.moe_layer_forward(ctypes.byref(xa), ctypes.byref(layer.router), ctypes.byref(layer.pool),
                                _ref(layer.shared), ctypes.byref(oa), ctypes.byref(opts), _stream_handle(stream))
    _check(st, "moe_layer_forward")
    return out


def moe_layer_forward_noalloc(layer: DeviceLayer, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                              path: str = "auto", out_dtype=torch.bfloat16, topk_ids: Optional[torch.Tensor] = None,
                              topk_w: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                              stream=None, input_rmsnorm_eps: float = 0.0) -> torch.Tensor:
    """moe_layer_forward on the library's fixed device scratch (no workspace).
    ``out`` must be given by callers that cannot allocate."""
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, layer.hidden), dtype=out_dtype, device=x.device)
    xa, oa = _act(x), _act(out)
    ptr = lambda t: None if t is None else t.data_ptr()
    opts = MqOpts(PATHS[path], ptr(topk_ids), ptr(topk_w), ptr(logits), None, 0, float(input_rmsnorm_eps), None)
    st = _lib.moe_layer_forward_noalloc(ctypes.byref(xa), ctypes.byref(layer.router), ctypes.byref(layer.pool),
                                        _ref(layer.shared), ctypes.byref(oa), ctypes.byref(opts),
                                        _stream_handle(stream))
    _check(st, "moe_layer_forward_noalloc")
    return out


def noalloc_scratch_bytes() -> int:
    return int(_lib.mq_noalloc_scratch_bytes())


class Stack:
    """Descriptor arrays of resident layers, all of one size, for moe_stack_forward."""

    def __init__(self, layers):
        self.layers = list(layers)
        n = len(self.layers)
        if n < 1:
            raise ValueError("a stack needs at least one layer")
        self.routers = (MqRouter * n)(*[l.router for l in self.layers])
        self.pools = (MqExpertPool * n)(*[l.pool for l in self.layers])
        has = [l.shared is not None for l in self.layers]
        if any(has) and not all(has):
            raise ValueError("either every layer of a stack has a shared expert or none has")
        self.shared = (MqShared * n)(*[l.shared for l in self.layers]) if all(has) else None
        first = self.layers[0]
        self.hidden, self.top_k, self.num_experts = first.hidden, first.top_k, first.num_experts

    def __len__(self) -> int:
        return len(self.layers)

    def workspace_bytes(self) -> int:
        n = _lib.mq_stack_workspace_bytes(self.routers, self.pools, self.shared, len(self))
        if n == 0:
            raise MoeError(MQ_ERR_SHAPE, "mq_stack_workspace_bytes")
        return int(n)

    def new_workspace(self, device="cuda") -> torch.Tensor:
        return torch.zeros(self.workspace_bytes(), dtype=torch.uint8, device=device)


def moe_stack_forward(stack: Stack, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, between_eps: float = 0.0,
                      input_rmsnorm_eps: float = 0.0, out_dtype=torch.bfloat16, path: str = "auto",
                      topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                      logits: Optional[torch.Tensor] = None, stream=None, tails=None) -> torch.Tensor:
    """One token through every layer of `stack` in one launch; layer l > 0
    takes bf16(out_{l-1}), RMS-normalised first when between_eps > 0.
    topk_ids / topk_w [n_layers][k] and logits [n_layers][E] are optional;
    ``tails`` is None or one Tail per layer."""
    if out is None:
        out = torch.empty((1, stack.hidden), dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = stack.new_workspace(x.device)
    xa, oa = _act(x), _act(out)
    ptr = lambda t: None if t is None else t.data_ptr()
    tarr = None
    if tails is not None:
        assert len(tails) == len(stack)
        tarr = (MqTail * len(stack))(*[t.struct for t in tails])
    opts = MqOpts(PATHS[path], ptr(topk_ids), ptr(topk_w), ptr(logits), workspace.data_ptr(), workspace.numel(),
                  float(input_rmsnorm_eps), None if tarr is None else ctypes.addressof(tarr))
    st = _lib.moe_stack_forward(ctypes.byref(xa), len(stack), stack.routers, stack.pools, stack.shared,
                                float(between_eps), ctypes.byref(oa), ctypes.byref(opts), _stream_handle(stream))
    _check(st, "moe_stack_forward")
    return out


def workspace_errors(workspace: torch.Tensor, stream=None) -> int:
    """Sticky error bits of the single-launch path in `workspace` (0: none)."""
    v = ctypes.c_uint32(0)
    _check(_lib.mq_workspace_errors(workspace.data_ptr(), workspace.numel(), ctypes.byref(v), _stream_handle(stream)),
           "mq_workspace_errors")
    return int(v.value)


def rmsnorm(x: torch.Tensor, out: Optional[torch.Tensor] = None, eps: float = 1e-6, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty_like(x)
    xa, oa = _act(x), _act(out)
    _check(_lib.mq_rmsnorm(ctypes.byref(xa), ctypes.byref(oa), eps, _stream_handle(stream)), "mq_rmsnorm")
    return out


def debug_unpack_codes(buf: torch.Tensor, rows: int, cols: int, bits: int, stream=None) -> torch.Tensor:
    out = torch.empty((rows, cols), dtype=torch.uint8, device=buf.device)
    d = MqQTensor(buf.data_ptr(), None, None, rows, cols, bits, GROUP, LAYOUT_DEV_V1)
    _check(_lib.mq_debug_unpack_codes(ctypes.byref(d), out.data_ptr(), _stream_handle(stream)),
           "mq_debug_unpack_codes")
    return out


def debug_dequant(buf: torch.Tensor, rows: int, cols: int, bits: int, stream=None) -> torch.Tensor:
    out = torch.empty((rows, cols), dtype=torch.float32, device=buf.device)
    d = MqQTensor(buf.data_ptr(), None, None, rows, cols, bits, GROUP, LAYOUT_DEV_V1)
    _check(_lib.mq_debug_dequant(ctypes.byref(d), out.data_ptr(), _stream_handle(stream)), "mq_debug_dequant")
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int, stream=None) -> None:
    """One streaming read of every byte of buf (a measurement kernel); sink int32 [workgroups]."""
    assert sink.numel() >= workgroups and sink.element_size() == 4
    _check(_lib.mq_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), workgroups,
                               _stream_handle(stream)), "mq_stream_read")


def qgemv(w_buf: torch.Tensor, rows: int, cols: int, bits: int, x: torch.Tensor, softcap: float = 0.0,
          want_y: bool = True, y_dtype=torch.float32, want_argmax: bool = True, workspace=None, stream=None):
    """y = W x (softcapped when softcap > 0) for bf16 token rows x [T][cols],
    with W a DEV_V1 device buffer; returns (y [T][rows] or None, argmax [T] or None)."""
    T = x.shape[0]
    d = MqQTensor(w_buf.data_ptr(), None, None, rows, cols, bits, GROUP, LAYOUT_DEV_V1)
    y = torch.empty((T, rows), dtype=y_dtype, device=x.device) if want_y else None
    am = torch.empty(T, dtype=torch.int32, device=x.device) if want_argmax else None
    if want_argmax and workspace is None:
        workspace = torch.empty(max(1, _lib.mq_qgemv_workspace_bytes(rows, T)), dtype=torch.uint8, device=x.device)
    xa = _act(x)
    ya = _act(y) if y is not None else None
    st = _lib.mq_qgemv(ctypes.byref(d), ctypes.byref(xa), _ref(ya), float(softcap),
                       None if am is None else am.data_ptr(), None if workspace is None else workspace.data_ptr(),
                       0 if workspace is None else workspace.numel(), _stream_handle(stream))
    _check(st, "mq_qgemv")
    return y, am


# ------------------------------------------------------------------ routing only, host-offloaded experts

def route(router_layer, x: torch.Tensor, ids: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
          logits: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Router, top-k and routing weights only (mq_route): (ids [T][k] int32, w [T][k] fp32)."""
    T = x.shape[0]
    k = router_layer.top_k
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(256, _lib.mq_route_workspace_bytes(ctypes.byref(router_layer.router), T)),
                                dtype=torch.uint8, device=x.device)
    xa = _act(x)
    _check(_lib.mq_route(ctypes.byref(xa), ctypes.byref(router_layer.router), ids.data_ptr(), w.data_ptr(),
                         None if logits is None else logits.data_ptr(), workspace.data_ptr(), workspace.numel(),
                         _stream_handle(stream)), "mq_route")
    return ids, w


class LfuCache:
    """The host slot cache of mq_lfu_* (state in a host buffer)."""

    def __init__(self, num_experts: int, num_slots: int):
        n = _lib.mq_lfu_state_bytes(num_experts, num_slots)
        if n == 0:
            raise MoeError(MQ_ERR_SHAPE, "mq_lfu_state_bytes")
        self.state = np.zeros((n + 7) // 8, dtype=np.uint64)
        self.nbytes = self.state.nbytes
        self.num_experts, self.num_slots = num_experts, num_slots
        _check(_lib.mq_lfu_init(self.state.ctypes.data, self.nbytes, num_experts, num_slots), "mq_lfu_init")

    def plan(self, ids: np.ndarray):
        """(slot of each id, [(expert, slot) to fill])."""
        ids = np.ascontiguousarray(ids, dtype=np.int32).ravel()
        n = ids.size
        slots = np.empty(n, np.int32)
        me, ms = np.empty(max(n, 1), np.int32), np.empty(max(n, 1), np.int32)
        nm = ctypes.c_int32(0)
        _check(_lib.mq_lfu_plan(self.state.ctypes.data, self.nbytes, ids.ctypes.data, n, slots.ctypes.data,
                                me.ctypes.data, ms.ctypes.data, ctypes.byref(nm)), "mq_lfu_plan")
        return slots, list(zip(me[:nm.value].tolist(), ms[:nm.value].tolist()))


class OffloadedLayer:
    """A layer whose routed experts stay in pinned host memory, with
    `num_slots` device slots managed by the LFU cache.  Each call routes the
    tokens on the GPU, reads the ids on the host, plans hits and misses,
    copies the missing experts into their slots on a copy stream (after the
    previous call's kernels, which own their slots until they finish), and
    runs the layer with that routing: the shared expert's kernels start at
    once and the routed experts' wait for the copies."""

    def __init__(self, src, num_slots: int = 16, device="cuda", max_tokens: int = 4, threads: int = 16):
        self.dev = DeviceLayer(src, device=device, resident_experts=False)
        d = self.dev
        E, stride = d.num_experts, d.pool.expert_stride
        self.stride = stride
        self.host_pool = torch.empty(E * stride, dtype=torch.uint8, pin_memory=True)
        hp = self.host_pool.numpy()

        def pack_expert(e):
            pack_expert_into(d.pool, e, src.gate.select(e), src.up.select(e), src.down.select(e), hp)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(pack_expert, range(E)))
        self.slot_buf = torch.empty(num_slots * stride, dtype=torch.uint8, device=device)
        d.pool.base = self.slot_buf.data_ptr()
        self.cache = LfuCache(E, num_slots)
        self.max_tokens, k = max_tokens, d.top_k
        self.ids = torch.empty((max_tokens, k), dtype=torch.int32, device=device)
        self.w = torch.empty((max_tokens, k), dtype=torch.float32, device=device)
        self.slots = torch.empty((max_tokens, k), dtype=torch.int32, device=device)
        self.ids_h = torch.empty(max_tokens * k, dtype=torch.int32, pin_memory=True)
        self.slots_h = torch.empty(max_tokens * k, dtype=torch.int32, pin_memory=True)
        self.route_ws = torch.empty(max(256, _lib.mq_route_workspace_bytes(ctypes.byref(d.router), max_tokens)),
                                    dtype=torch.uint8, device=device)
        self.workspace = d.new_workspace(max_tokens)
        self.copy_stream = torch.cuda.Stream(device=device)
        self.ready = torch.cuda.Event()
        self.done = torch.cuda.Event()
        self.done.record()
        self.hits = self.misses = 0

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                tail: Optional[Tail] = None, input_rmsnorm_eps: float = 0.0) -> torch.Tensor:
        T = x.shape[0]
        k = self.dev.top_k
        assert 0 < T <= self.max_tokens
        s = torch.cuda.current_stream()
        ids, w, slots = self.ids[:T], self.w[:T], self.slots[:T]
        if input_rmsnorm_eps > 0:
            # the router sees the same normalised rows as the experts
            xr = rmsnorm(x, eps=input_rmsnorm_eps)
        else:
            xr = x
        route(self.dev, xr, ids, w, workspace=self.route_ws)
        self.ids_h[:T * k].copy_(ids.view(-1), non_blocking=True)
        s.synchronize()                                   # the host reads the expert ids
        slot_of, fills = self.cache.plan(self.ids_h[:T * k].numpy())
        self.misses += len(fills)
        self.hits += len(set(self.ids_h[:T * k].tolist())) - len(fills)
        cs = self.copy_stream
        cs.wait_event(self.done)                          # earlier kernels own their slots until done
        with torch.cuda.stream(cs):
            for e, sl in fills:
                self.slot_buf[sl * self.stride:(sl + 1) * self.stride].copy_(
                    self.host_pool[e * self.stride:(e + 1) * self.stride], non_blocking=True)
            self.ready.record(cs)
        self.slots_h[:T * k] = torch.from_numpy(slot_of)
        slots.view(-1).copy_(self.slots_h[:T * k], non_blocking=True)
        out = moe_layer_forward(self.dev, x, out=out, workspace=self.workspace, path="gemv", out_dtype=out_dtype,
                                tail=tail, input_rmsnorm_eps=input_rmsnorm_eps, route_ids=ids, route_w=w,
                                route_slots=slots, experts_ready=self.ready)
        self.done.record(s)
        return out

"""quantized_moe_ffn_amd — routed MoE FFN over GGUF block-quantized experts on MI355X.

A thin Python binding over ``libmoe.so`` (C ABI in ``include/moe.h``).  Every
function here only marshals arguments: torch tensors supply device memory and
the current HIP stream, and every step of the path runs in the library's HIP
kernels.  There is no CPU fallback: if ``libmoe.so`` is missing or cannot be
loaded, the first call raises.

Entry points keep the C names: ``moe_route_topk``, ``moe_quantize_act``,
``moe_router_logits``, ``moe_expert_ffn_q``, ``moe_combine``, ``moe_combine_ep``, ``moe_shared_gate``,
``moe_forward``, ``moe_forward_ep``, ``moe_forward_noalloc``, ``moe_forward_router``, ``moe_dequant_q``,
``moe_check_device_errors``, ``moe_last_error``, ``moe_abi_version``,
``moe_route_workspace_bytes``, ``moe_ffn_workspace_bytes``,
``moe_forward_workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_Q8_0 = 8
MOE_Q4_K = 12
MOE_Q5_K = 13
MOE_Q5_1 = 7
MOE_ROUTE_RENORM = 1
MOE_FFN_AUTO = 0
AUTO_DECODE_MAX_T = 8   # MOE_FFN_AUTO takes the fp-activation path up to this many tokens
MOE_FFN_DECODE = 1
MOE_FFN_INT8 = 2
MOE_FFN_PAIR_BF16 = 16  # layer calls: per-pair outputs stay in the workspace (bf16 on the MFMA GEMMs)

BLOCK_WEIGHTS = {MOE_Q4_K: 256, MOE_Q5_K: 256, MOE_Q8_0: 32, MOE_Q5_1: 32}
BLOCK_BYTES = {MOE_Q4_K: 144, MOE_Q5_K: 176, MOE_Q8_0: 34, MOE_Q5_1: 24}

EXPORTS = (
    "moe_abi_version", "moe_last_error", "moe_route_workspace_bytes", "moe_route_topk",
    "moe_quantize_act", "moe_ffn_workspace_bytes", "moe_expert_ffn_q", "moe_combine",
    "moe_dequant_q", "moe_check_device_errors", "moe_forward_workspace_bytes", "moe_forward",
    "moe_router_logits", "moe_combine_ep", "moe_shared_gate", "moe_forward_ep", "moe_forward_noalloc",
    "moe_forward_router",
)

MOE_NOALLOC_SCRATCH_BYTES = 8 << 20   # the static workspace of moe_forward_noalloc, per GPU


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__("%s failed with status %d: %s" % (where, status, message))
        self.status = status


class moe_qmatrix(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("qtype", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("row_bytes", ctypes.c_int64), ("expert_bytes", ctypes.c_int64)]


class moe_layer(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("has_shared", ctypes.c_int32), ("gate", moe_qmatrix), ("up", moe_qmatrix),
                ("down", moe_qmatrix), ("sh_gate", moe_qmatrix), ("sh_up", moe_qmatrix),
                ("sh_down", moe_qmatrix)]


class moe_epilogue(ctypes.Structure):
    _fields_ = [("residual", ctypes.c_void_p), ("shared_gate", ctypes.c_void_p)]


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("idx", "w", "count", "offset", "pair", "active", "n_active")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libmoe.so and declares its signatures (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmoe.so not found at %s: build it first (python -m quantized_moe_ffn_amd.build "
                           "or __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    P, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    st = ctypes.c_int
    lib.moe_abi_version.restype = i32
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_route_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_route_workspace_bytes.restype = sz
    lib.moe_route_topk.argtypes = [P, i32, i32, i32, u32, ctypes.POINTER(moe_routing), P, sz, P]
    lib.moe_route_topk.restype = st
    lib.moe_quantize_act.argtypes = [P, i32, i32, P, P, P]
    lib.moe_quantize_act.restype = st
    lib.moe_router_logits.argtypes = [P, i32, i32, P, i32, P, P]
    lib.moe_router_logits.restype = st
    lib.moe_ffn_workspace_bytes.argtypes = [ctypes.POINTER(moe_layer), i32, i32, u32]
    lib.moe_ffn_workspace_bytes.restype = sz
    lib.moe_expert_ffn_q.argtypes = [ctypes.POINTER(moe_layer), ctypes.POINTER(moe_routing), i32, i32, P, P, P,
                                     u32, P, P, P, sz, P]
    lib.moe_expert_ffn_q.restype = st
    lib.moe_combine.argtypes = [P, P, P, P, i32, i32, i32, P, P]
    lib.moe_combine.restype = st
    lib.moe_dequant_q.argtypes = [P, i32, i64, P, P]
    lib.moe_dequant_q.restype = st
    lib.moe_forward_workspace_bytes.argtypes = [ctypes.POINTER(moe_layer), i32, i32, u32]
    lib.moe_forward_workspace_bytes.restype = sz
    lib.moe_forward.argtypes = [ctypes.POINTER(moe_layer), P, P, i32, i32, u32, u32, ctypes.POINTER(moe_routing),
                                P, P, P, P, P, sz, P]
    lib.moe_forward.restype = st
    lib.moe_forward_ep.argtypes = [ctypes.POINTER(moe_layer), P, P, i32, i32, u32, u32,
                                   ctypes.POINTER(moe_routing), P, P, P, ctypes.POINTER(moe_epilogue), P, P, sz, P]
    lib.moe_forward_ep.restype = st
    lib.moe_forward_noalloc.argtypes = [ctypes.POINTER(moe_layer), P, P, i32, i32, u32, u32,
                                        ctypes.POINTER(moe_routing), P, P, P, P, P]
    lib.moe_forward_noalloc.restype = st
    lib.moe_forward_router.argtypes = [ctypes.POINTER(moe_layer), P, P, P, i32, i32, u32, u32,
                                       ctypes.POINTER(moe_routing), P, P, P, P, P, sz, P]
    lib.moe_forward_router.restype = st
    lib.moe_combine_ep.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, P]
    lib.moe_combine_ep.restype = st
    lib.moe_shared_gate.argtypes = [P, i32, i32, P, P, P]
    lib.moe_shared_gate.restype = st
    lib.moe_check_device_errors.argtypes = [P]
    lib.moe_check_device_errors.restype = st
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where, moe_last_error())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ----------------------------------------------------------------------------- descriptors

class QMatrix:
    """A device bank of quantized matrices: uint8 tensor [n_experts][rows][row_bytes]."""

    def __init__(self, data, qtype: int, cols: int):
        assert data.dtype.itemsize == 1 and data.dim() == 3 and data.is_contiguous()
        self.data, self.qtype, self.cols = data, int(qtype), int(cols)
        self.rows = data.shape[1]
        self.row_bytes = cols // BLOCK_WEIGHTS[qtype] * BLOCK_BYTES[qtype]
        assert data.shape[2] == self.row_bytes, (data.shape, self.row_bytes)

    def struct(self) -> moe_qmatrix:
        return moe_qmatrix(self.data.data_ptr(), self.qtype, self.rows, self.cols, 0, self.row_bytes,
                           self.data.shape[1] * self.data.shape[2])


class Layer:
    """One MoE layer: routed banks gate/up [E][I][.], down [E][H][.], optional shared expert."""

    def __init__(self, gate: QMatrix, up: QMatrix, down: QMatrix, shared=None):
        self.gate, self.up, self.down, self.shared = gate, up, down, shared
        self.n_experts = gate.data.shape[0]
        self.hidden = gate.cols
        self.inter = gate.rows
        s = moe_layer()
        s.n_experts, s.hidden, s.inter = self.n_experts, self.hidden, self.inter
        s.gate, s.up, s.down = gate.struct(), up.struct(), down.struct()
        if shared is not None:
            s.has_shared = 1
            s.sh_gate, s.sh_up, s.sh_down = (m.struct() for m in shared)
        self._s = s

    def struct(self) -> moe_layer:
        return self._s


class Routing:
    """Device buffers written by moe_route_topk for T tokens, E experts, top-k."""

    def __init__(self, T: int, E: int, k: int, device="cuda"):
        import torch
        i32 = dict(dtype=torch.int32, device=device)
        self.T, self.E, self.k = T, E, k
        self.idx = torch.empty((T, k), **i32)
        self.w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.count = torch.empty(E, **i32)
        self.offset = torch.empty(E + 1, **i32)
        self.pair = torch.empty(T * k, **i32)
        self.active = torch.empty(max(1, min(E, T * k)), **i32)
        self.n_active = torch.empty(1, **i32)
        self._s = moe_routing(*(t.data_ptr() for t in (self.idx, self.w, self.count, self.offset, self.pair,
                                                        self.active, self.n_active)))

    def struct(self) -> moe_routing:
        return self._s


# ----------------------------------------------------------------------------- C entry points

def moe_abi_version() -> int:
    return int(load_library().moe_abi_version())


def moe_last_error() -> str:
    return load_library().moe_last_error().decode()


def moe_route_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(load_library().moe_route_workspace_bytes(T, E, k))


def moe_route_topk(logits, k: int, routing: Routing, renorm: bool = True, workspace=None, stream=None):
    T, E = logits.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().moe_route_topk(_ptr(logits), T, E, k, MOE_ROUTE_RENORM if renorm else 0,
                                       ctypes.byref(routing.struct()), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "moe_route_topk")


def moe_router_logits(x, w_router, logits, stream=None):
    """logits[t][e] = sum_h w_router[e][h] * x[t][h] (fp32 device tensors)."""
    T, H = x.shape
    E = w_router.shape[0]
    assert w_router.shape[1] == H and tuple(logits.shape) == (T, E)
    _check(load_library().moe_router_logits(_ptr(x), T, H, _ptr(w_router), E, _ptr(logits), _stream(stream)),
           "moe_router_logits")


def moe_quantize_act(x, xq, xd, stream=None):
    T, H = x.shape
    _check(load_library().moe_quantize_act(_ptr(x), T, H, _ptr(xq), _ptr(xd), _stream(stream)),
           "moe_quantize_act")


def moe_ffn_workspace_bytes(layer: Layer, T: int, k: int, flags: int = MOE_FFN_AUTO) -> int:
    return int(load_library().moe_ffn_workspace_bytes(ctypes.byref(layer.struct()), T, k, flags))


def moe_expert_ffn_q(layer: Layer, routing: Routing, T: int, k: int, y_pair, x=None, xq=None, xd=None,
                     flags: int = MOE_FFN_AUTO, y_shared=None, workspace=None, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().moe_expert_ffn_q(ctypes.byref(layer.struct()), ctypes.byref(routing.struct()), T, k,
                                         _ptr(x), _ptr(xq), _ptr(xd), flags, _ptr(y_pair), _ptr(y_shared),
                                         _ptr(workspace), nbytes, _stream(stream))
    _check(st, "moe_expert_ffn_q")


def moe_combine(y_pair, w, out, y_shared=None, shared_scale=None, stream=None):
    T, k = w.shape
    H = out.shape[1]
    _check(load_library().moe_combine(_ptr(y_pair), _ptr(w), _ptr(y_shared), _ptr(shared_scale), T, k, H,
                                      _ptr(out), _stream(stream)), "moe_combine")


def moe_combine_ep(y_pair, w, out, y_shared=None, shared_scale=None, shared_gate_s=None, residual=None,
                   stream=None):
    T, k = w.shape
    H = out.shape[1]
    _check(load_library().moe_combine_ep(_ptr(y_pair), _ptr(w), _ptr(y_shared), _ptr(shared_scale),
                                         _ptr(shared_gate_s), _ptr(residual), T, k, H, _ptr(out),
                                         _stream(stream)), "moe_combine_ep")


def moe_shared_gate(x, gate_w, s, stream=None):
    """s[t] = sigmoid(gate_w . x[t]) (fp32 device tensors)."""
    T, H = x.shape
    _check(load_library().moe_shared_gate(_ptr(x), T, H, _ptr(gate_w), _ptr(s), _stream(stream)),
           "moe_shared_gate")


def moe_dequant_q(blocks, qtype: int, n_weights: int, out, stream=None):
    _check(load_library().moe_dequant_q(_ptr(blocks), qtype, n_weights, _ptr(out), _stream(stream)),
           "moe_dequant_q")


def moe_forward_workspace_bytes(layer: Layer, T: int, k: int, flags: int = MOE_FFN_AUTO) -> int:
    return int(load_library().moe_forward_workspace_bytes(ctypes.byref(layer.struct()), T, k, flags))


def moe_forward(layer: Layer, logits, x, k: int, routing: Routing, y_pair, out, y_shared=None, shared_scale=None,
                renorm: bool = True, flags: int = MOE_FFN_AUTO, workspace=None, stream=None):
    T = x.shape[0]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().moe_forward(ctypes.byref(layer.struct()), _ptr(logits), _ptr(x), T, k,
                                    MOE_ROUTE_RENORM if renorm else 0, flags, ctypes.byref(routing.struct()),
                                    _ptr(y_pair), _ptr(y_shared), _ptr(shared_scale), _ptr(out), _ptr(workspace),
                                    nbytes, _stream(stream))
    _check(st, "moe_forward")


def moe_forward_ep(layer: Layer, logits, x, k: int, routing: Routing, y_pair, out, y_shared=None,
                   shared_scale=None, residual=None, shared_gate=None, renorm: bool = True,
                   flags: int = MOE_FFN_AUTO, workspace=None, stream=None):
    T = x.shape[0]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ep = moe_epilogue(_ptr(residual), _ptr(shared_gate))
    st = load_library().moe_forward_ep(ctypes.byref(layer.struct()), _ptr(logits), _ptr(x), T, k,
                                       MOE_ROUTE_RENORM if renorm else 0, flags, ctypes.byref(routing.struct()),
                                       _ptr(y_pair), _ptr(y_shared), _ptr(shared_scale), ctypes.byref(ep), _ptr(out),
                                       _ptr(workspace), nbytes, _stream(stream))
    _check(st, "moe_forward_ep")


def moe_forward_noalloc(layer: Layer, logits, x, k: int, routing: Routing, y_pair, out, y_shared=None,
                        shared_scale=None, renorm: bool = True, flags: int = MOE_FFN_AUTO, stream=None):
    """moe_forward with the library's static per-GPU scratch as its workspace (no allocation)."""
    T = x.shape[0]
    st = load_library().moe_forward_noalloc(ctypes.byref(layer.struct()), _ptr(logits), _ptr(x), T, k,
                                            MOE_ROUTE_RENORM if renorm else 0, flags, ctypes.byref(routing.struct()),
                                            _ptr(y_pair), _ptr(y_shared), _ptr(shared_scale), _ptr(out),
                                            _stream(stream))
    _check(st, "moe_forward_noalloc")


def moe_forward_router(layer: Layer, x, w_router, logits, k: int, routing: Routing, y_pair, out, workspace,
                       y_shared=None, shared_scale=None, renorm: bool = True, flags: int = MOE_FFN_AUTO, stream=None):
    """The layer from x and the router matrix (logits written); moe_forward's workspace."""
    T = x.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().moe_forward_router(ctypes.byref(layer.struct()), _ptr(x), _ptr(w_router), _ptr(logits), T, k,
                                           MOE_ROUTE_RENORM if renorm else 0, flags, ctypes.byref(routing.struct()),
                                           _ptr(y_pair), _ptr(y_shared), _ptr(shared_scale), _ptr(out),
                                           _ptr(workspace), nbytes, _stream(stream))
    _check(st, "moe_forward_router")


def moe_check_device_errors(stream=None):
    _check(load_library().moe_check_device_errors(_stream(stream)), "moe_check_device_errors")


# ----------------------------------------------------------------------------- whole layer

class LayerBuffers:
    """Routing, workspace and output buffers for one (T, k) shape of a layer."""

    def __init__(self, layer: Layer, T: int, k: int, flags: int = MOE_FFN_AUTO, device="cuda"):
        import torch
        H, E = layer.hidden, layer.n_experts
        self.T, self.k, self.flags = T, k, flags
        self.routing = Routing(T, E, k, device)
        rw = moe_route_workspace_bytes(T, E, k)
        self.route_ws = torch.empty(max(rw, 1), dtype=torch.uint8, device=device)
        fw = moe_ffn_workspace_bytes(layer, T, k, flags & ~MOE_FFN_PAIR_BF16)
        self.ffn_ws = torch.empty(max(fw, 256), dtype=torch.uint8, device=device)
        self.y_pair = torch.empty((T * k, H), dtype=torch.float32, device=device)
        self.y_shared = torch.empty((T, H), dtype=torch.float32, device=device) if layer.shared else None
        self.xq = torch.empty((T, H), dtype=torch.int8, device=device)
        self.xd = torch.empty((T, H // 256), dtype=torch.float32, device=device)
        self.out = torch.empty((T, H), dtype=torch.float32, device=device)
        self.gate_s = torch.empty(T, dtype=torch.float32, device=device)
        fwd = moe_forward_workspace_bytes(layer, T, k, flags)
        self.fwd_ws = torch.empty(max(fwd, 256), dtype=torch.uint8, device=device)


def forward(layer: Layer, logits, x, k: int, bufs: LayerBuffers | None = None, flags: int = MOE_FFN_AUTO,
            renorm: bool = True, shared_scale=None, stream=None, fused: bool = True, residual=None,
            shared_gate=None) -> LayerBuffers:
    """The whole layer on one stream.  fused=True: one moe_forward call (two kernels
    for decode batches), moe_forward_ep when an epilogue (residual, shared-expert
    gate vector) is given; fused=False: the separate calls route -> (quantize) ->
    expert FFN -> (shared gate) -> combine."""
    T = x.shape[0]
    if bufs is None:
        bufs = LayerBuffers(layer, T, k, flags, device=x.device)
    epilogue = residual is not None or shared_gate is not None
    if fused:
        if epilogue:
            moe_forward_ep(layer, logits, x, k, bufs.routing, bufs.y_pair, bufs.out, bufs.y_shared, shared_scale,
                           residual, shared_gate, renorm, flags, bufs.fwd_ws, stream)
        else:
            moe_forward(layer, logits, x, k, bufs.routing, bufs.y_pair, bufs.out, bufs.y_shared, shared_scale,
                        renorm, flags, bufs.fwd_ws, stream)
        return bufs
    sel = flags & ~MOE_FFN_PAIR_BF16   # the separate stages hand fp32 y_pair to the combine
    path = sel if sel != MOE_FFN_AUTO else (MOE_FFN_DECODE if T <= AUTO_DECODE_MAX_T else MOE_FFN_INT8)
    moe_route_topk(logits, k, bufs.routing, renorm, bufs.route_ws, stream)
    if path == MOE_FFN_INT8:
        moe_quantize_act(x, bufs.xq, bufs.xd, stream)
    moe_expert_ffn_q(layer, bufs.routing, T, k, bufs.y_pair, x=x if path == MOE_FFN_DECODE else None,
                     xq=bufs.xq if path == MOE_FFN_INT8 else None, xd=bufs.xd if path == MOE_FFN_INT8 else None,
                     flags=path, y_shared=bufs.y_shared, workspace=bufs.ffn_ws, stream=stream)
    if epilogue:
        sg = None
        if shared_gate is not None:
            sg = bufs.gate_s
            moe_shared_gate(x, shared_gate, sg, stream)
        moe_combine_ep(bufs.y_pair, bufs.routing.w, bufs.out, bufs.y_shared, shared_scale, sg, residual, stream)
    else:
        moe_combine(bufs.y_pair, bufs.routing.w, bufs.out, bufs.y_shared, shared_scale, stream)
    return bufs

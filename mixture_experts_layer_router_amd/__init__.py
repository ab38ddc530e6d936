"""Python binding of lc_moe (liblc_moe.so): argument marshalling only.

Every step of the layer runs in the HIP library; this module converts torch tensors to
device pointers and the current torch stream to a hipStream_t, checks tensor
dtype/shape/device, and turns an error status into an exception.  torch is used only for
device memory and streams.  The library is opened on first use and a missing build raises at once
(``python -m mixture_experts_layer_router_amd.build``); there is no fallback path.

Low-level entry points carry the C names (``lc_moe_route``, ``lc_moe_expert_load``,
``lc_moe_permute``, ``lc_moe_forward``, ``lc_moe_forward_staged``, ``lc_moe_forward_noalloc``,
``lc_moe_ffn_backward``, ``lc_moe_backward_workspace_size``, ``lc_moe_bias_update``,
``lc_moe_quantize_weights``, ``lc_moe_quantize_activations``, ``lc_moe_fp8_weights_size``,
``lc_moe_pack_weights``,
``lc_moe_packed_weights_size``, ``lc_moe_workspace_size``); ``route``, ``expert_load``,
``permute``, ``forward``, ``bias_update``, ``quantize_weights``, ``quantize_activations`` and
``pack_weights``
allocate outputs and a workspace with torch where needed and call them.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblc_moe.so")

# torch must be loaded first: its wheel ships its own HIP runtime with the same soname
# (libamdhip64.so.7).  Loaded in this order, liblc_moe.so binds to that runtime and the
# process holds one HIP runtime; the other order would load two.
import torch  # noqa: E402,F401

F32, BF16 = 0, 1
NUM_STAGES = 5
STATUS = {0: "ok", 1: "E_NULLPTR", 2: "E_SHAPE", 3: "E_DTYPE", 4: "E_ALIGN", 5: "E_WORKSPACE",
          6: "E_DEVICE"}


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
                ("Z", ctypes.c_int32), ("K", ctypes.c_int32), ("I", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("fp8", ctypes.c_void_p), ("packed", ctypes.c_void_p),
                ("fp8_act", ctypes.c_int32)]


class Pid(ctypes.Structure):
    _fields_ = [("kp", ctypes.c_float), ("ki", ctypes.c_float), ("kd", ctypes.c_float)]


_vp, _sz = ctypes.c_void_p, ctypes.c_size_t
_SIG = {
    "lc_moe_workspace_size": (_sz, [ctypes.POINTER(Shape)]),
    "lc_moe_route": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lc_moe_expert_load": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _sz, _vp]),
    "lc_moe_permute": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _sz, _vp]),
    "lc_moe_forward": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, ctypes.POINTER(Weights), _vp,
                                      _vp, _vp, _vp, _vp, _sz, _vp]),
    "lc_moe_forward_staged": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, ctypes.POINTER(Weights),
                                             _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "lc_moe_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, ctypes.POINTER(Weights), _vp,
                                              _vp, _vp, _vp, _vp]),
    "lc_moe_backward_workspace_size": (_sz, [ctypes.POINTER(Shape)]),
    "lc_moe_ffn_backward": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, ctypes.POINTER(Weights), _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lc_moe_fp8_weights_size": (_sz, [ctypes.POINTER(Shape)]),
    "lc_moe_quantize_weights": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _sz, _vp]),
    "lc_moe_quantize_activations": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp]),
    "lc_moe_packed_weights_size": (_sz, [ctypes.POINTER(Shape)]),
    "lc_moe_pack_weights": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _sz, _vp]),
    "lc_moe_bias_update": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(Pid), _vp, _vp,
                                          _vp, _vp, _vp, _vp]),
    "lc_moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "lc_moe_stage_name": (ctypes.c_char_p, [ctypes.c_int]),
}
_LIB = None


def lib():
    """The loaded liblc_moe.so (opened on first use; raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m mixture_experts_layer_router_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(handle, name)
            f.restype, f.argtypes = res, args
        _LIB = handle
    return _LIB


EXPORTED = tuple(_SIG)


class LcMoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({lib().lc_moe_status_str(status).decode()})")


def _check(status: int, where: str):
    if status != 0:
        raise LcMoeError(status, where)


def status_str(status: int) -> str:
    return lib().lc_moe_status_str(status).decode()


def stage_name(i: int) -> str:
    return lib().lc_moe_stage_name(i).decode()


def make_shape(T, d, N, Z, K, I, dtype) -> Shape:
    if not isinstance(dtype, int):
        import torch
        dtype = BF16 if dtype == torch.bfloat16 else F32 if dtype == torch.float32 else -1
    return Shape(T, d, N, Z, K, I, dtype)


def lc_moe_workspace_size(shape: Shape) -> int:
    return int(lib().lc_moe_workspace_size(ctypes.byref(shape)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ---- low-level: same names and argument order as the C-ABI ------------------------------

def lc_moe_route(shape, x, w_router, bias, topk_idx, topk_gate, workspace, stream=None):
    _check(lib().lc_moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(bias),
                             _ptr(topk_idx), _ptr(topk_gate), _ptr(workspace), _nbytes(workspace),
                             _stream(stream)), "lc_moe_route")


def lc_moe_expert_load(shape, topk_idx, load, ffn_per_token, workspace, stream=None):
    _check(lib().lc_moe_expert_load(ctypes.byref(shape), _ptr(topk_idx), _ptr(load),
                                   _ptr(ffn_per_token), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream)), "lc_moe_expert_load")


def lc_moe_permute(shape, x, topk_idx, ffn_offsets, perm_token, slot_row, x_perm, load,
                   workspace, stream=None):
    _check(lib().lc_moe_permute(ctypes.byref(shape), _ptr(x), _ptr(topk_idx), _ptr(ffn_offsets),
                               _ptr(perm_token), _ptr(slot_row), _ptr(x_perm), _ptr(load),
                               _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "lc_moe_permute")


def _weights(w_router, bias, w_gate, w_up, w_down, fp8=None, packed=None, fp8_act=False) -> Weights:
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    w = Weights(p(w_router), p(bias), p(w_gate), p(w_up), p(w_down), p(fp8), p(packed), int(bool(fp8_act)))
    # the struct holds raw device addresses: keep the tensors alive as long as it lives, or
    # a tensor made inline would go back to torch's allocator and be handed out again
    w._tensors = (w_router, bias, w_gate, w_up, w_down, fp8, packed)
    return w


def lc_moe_fp8_weights_size(shape: Shape) -> int:
    return int(lib().lc_moe_fp8_weights_size(ctypes.byref(shape)))


def lc_moe_quantize_weights(shape, w_gate, w_up, w_down, fp8_weights, stream=None):
    _check(lib().lc_moe_quantize_weights(ctypes.byref(shape), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                        _ptr(fp8_weights), _nbytes(fp8_weights), _stream(stream)),
           "lc_moe_quantize_weights")


def lc_moe_quantize_activations(x, rows, cols, codes, scales, stream=None):
    _check(lib().lc_moe_quantize_activations(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)),
           "lc_moe_quantize_activations")


def lc_moe_packed_weights_size(shape: Shape) -> int:
    return int(lib().lc_moe_packed_weights_size(ctypes.byref(shape)))


def lc_moe_pack_weights(shape, w_gate, w_up, w_down, packed_weights, stream=None):
    _check(lib().lc_moe_pack_weights(ctypes.byref(shape), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                    _ptr(packed_weights), _nbytes(packed_weights), _stream(stream)),
           "lc_moe_pack_weights")


def lc_moe_forward(shape, x, weights: Weights, y, topk_idx, topk_gate, load, workspace,
                   stream=None):
    _check(lib().lc_moe_forward(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(y),
                               _ptr(topk_idx), _ptr(topk_gate), _ptr(load), _ptr(workspace),
                               _nbytes(workspace), _stream(stream)), "lc_moe_forward")


STATIC_WORKSPACE_BYTES = 128 << 20   # LC_MOE_STATIC_WORKSPACE_BYTES


def lc_moe_forward_noalloc(shape, x, weights: Weights, y, topk_idx, topk_gate, load, stream=None):
    _check(lib().lc_moe_forward_noalloc(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(y),
                                       _ptr(topk_idx), _ptr(topk_gate), _ptr(load), _stream(stream)),
           "lc_moe_forward_noalloc")


def lc_moe_forward_staged(shape, x, weights: Weights, y, topk_idx, topk_gate, load, workspace,
                          stream=None, stage_events=None):
    arr = None
    if stage_events is not None:
        arr = (ctypes.c_void_p * len(stage_events))(*[e.cuda_event for e in stage_events])
    _check(lib().lc_moe_forward_staged(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(y),
                                      _ptr(topk_idx), _ptr(topk_gate), _ptr(load), _ptr(workspace),
                                      _nbytes(workspace), _stream(stream),
                                      ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None),
           "lc_moe_forward_staged")


def lc_moe_backward_workspace_size(shape: Shape) -> int:
    return int(lib().lc_moe_backward_workspace_size(ctypes.byref(shape)))


def lc_moe_ffn_backward(shape, x, weights: Weights, topk_idx, topk_gate, dy, dx, dw_gate, dw_up, dw_down,
                        workspace, stream=None):
    _check(lib().lc_moe_ffn_backward(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(topk_idx),
                                    _ptr(topk_gate), _ptr(dy), _ptr(dx), _ptr(dw_gate), _ptr(dw_up),
                                    _ptr(dw_down), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "lc_moe_ffn_backward")


def lc_moe_bias_update(shape, gains: Pid, load, target, bias, integral, prev_err, stream=None):
    _check(lib().lc_moe_bias_update(ctypes.byref(shape), ctypes.byref(gains), _ptr(load),
                                   _ptr(target), _ptr(bias), _ptr(integral), _ptr(prev_err),
                                   _stream(stream)), "lc_moe_bias_update")


# ---- convenience wrappers: allocate outputs with torch, then call the C entry point -----

def _shape_of(x, N, Z, K, I):
    T, d = x.shape
    return make_shape(T, d, N, Z, K, I, x.dtype)


def workspace_for(shape: Shape, device):
    import torch
    n = lc_moe_workspace_size(shape)
    if n == 0:
        raise LcMoeError(2, "lc_moe_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def route(x, w_router, bias, K, N, workspace=None):
    """(topk_idx int32 [T,K], topk_gate fp32 [T,K])."""
    import torch
    E = w_router.shape[0]
    shape = _shape_of(x, N, E - N, K, 8)
    ws = workspace if workspace is not None else workspace_for(shape, x.device)
    idx = torch.empty((x.shape[0], K), dtype=torch.int32, device=x.device)
    gate = torch.empty((x.shape[0], K), dtype=torch.float32, device=x.device)
    lc_moe_route(shape, x, w_router, bias, idx, gate, ws)
    return idx, gate


def expert_load(topk_idx, N, E, workspace=None, d=8, dtype=BF16):
    """(load int32 [E], ffn_per_token int32 [T])."""
    import torch
    T, K = topk_idx.shape
    shape = make_shape(T, d, N, E - N, K, 8, dtype)
    ws = workspace if workspace is not None else workspace_for(shape, topk_idx.device)
    load = torch.empty(E, dtype=torch.int32, device=topk_idx.device)
    ffn = torch.empty(T, dtype=torch.int32, device=topk_idx.device)
    lc_moe_expert_load(shape, topk_idx, load, ffn, ws)
    return load, ffn


def permute(x, topk_idx, N, E, with_x_perm=True, workspace=None):
    """dict(ffn_offsets, perm_token, slot_row, x_perm, load)."""
    import torch
    T, K = topk_idx.shape
    shape = make_shape(T, x.shape[1], N, E - N, K, 8, x.dtype)
    ws = workspace if workspace is not None else workspace_for(shape, x.device)
    dev = x.device
    out = dict(ffn_offsets=torch.empty(N + 1, dtype=torch.int32, device=dev),
               perm_token=torch.full((T * K,), -7, dtype=torch.int32, device=dev),
               slot_row=torch.empty((T, K), dtype=torch.int32, device=dev),
               x_perm=torch.empty((T * K, x.shape[1]), dtype=x.dtype, device=dev) if with_x_perm else None,
               load=torch.empty(E, dtype=torch.int32, device=dev))
    lc_moe_permute(shape, x, topk_idx, out["ffn_offsets"], out["perm_token"], out["slot_row"],
                   out["x_perm"], out["load"], ws)
    return out


def forward(x, w_router, bias, w_gate, w_up, w_down, K, workspace=None, stage_events=None, fp8=None,
            packed=None, fp8_act=False):
    """dict(y, topk_idx, topk_gate, load); x [T,d]; w_gate/w_up [N,I,d]; w_down [N,d,I];
    fp8: optional block-FP8 weights from quantize_weights (then used instead);
    packed: optional packed bf16 weights from pack_weights (then read instead);
    fp8_act: with fp8, quantize x and H to block FP8 too (FP8 matrix cores)."""
    import torch
    N, I, _ = w_gate.shape
    E = w_router.shape[0]
    shape = _shape_of(x, N, E - N, K, I)
    ws = workspace if workspace is not None else workspace_for(shape, x.device)
    T, dev = x.shape[0], x.device
    y = torch.empty_like(x)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    load = torch.empty(E, dtype=torch.int32, device=dev)
    wts = _weights(w_router, bias, w_gate, w_up, w_down, fp8, packed, fp8_act)
    if stage_events is None:
        lc_moe_forward(shape, x, wts, y, idx, gate, load, ws)
    else:
        lc_moe_forward_staged(shape, x, wts, y, idx, gate, load, ws, stage_events=stage_events)
    return dict(y=y, topk_idx=idx, topk_gate=gate, load=load)


def ffn_backward(x, w_gate, w_up, w_down, topk_idx, topk_gate, dy, Z, workspace=None):
    """dict(dx, dw_gate, dw_up, dw_down): gradients of sum <dy, y> for the forward's picks
    and gates (held fixed); x, dy [T,d] bf16; w_gate/w_up [N,I,d]; w_down [N,d,I]; Z = number
    of zero-computation experts of the layer."""
    import torch
    N, I, d = w_gate.shape
    T, K = topk_idx.shape
    shape = make_shape(T, d, N, Z, K, I, x.dtype)
    if workspace is None:
        n = lc_moe_backward_workspace_size(shape)
        if n == 0:
            raise LcMoeError(2, "lc_moe_backward_workspace_size")
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    out = dict(dx=torch.empty_like(x), dw_gate=torch.empty_like(w_gate), dw_up=torch.empty_like(w_up),
               dw_down=torch.empty_like(w_down))
    wts = _weights(None, None, w_gate, w_up, w_down)
    lc_moe_ffn_backward(shape, x, wts, topk_idx, topk_gate, dy, out["dx"], out["dw_gate"], out["dw_up"],
                        out["dw_down"], workspace)
    return out


def bias_update(load, target, bias, integral, prev_err, T, K, N, kp, ki, kd):
    """One PID update of bias, integral and prev_err (all fp32 [E], updated in place) from
    the int32 [E] loads of a step of T tokens with K picks each."""
    E = load.shape[0]
    shape = make_shape(T, 8, N, E - N, K, 8, BF16)
    lc_moe_bias_update(shape, Pid(kp, ki, kd), load, target, bias, integral, prev_err)


def quantize_weights(w_gate, w_up, w_down):
    """Block-FP8 form of bf16 expert weights (W_gate, W_up [N,I,d], W_down [N,d,I]) as a
    uint8 device tensor, for ``forward(..., fp8=...)`` / ``Weights.fp8``."""
    import torch
    N, I, d = w_gate.shape
    shape = make_shape(1, d, N, 0, 1, I, BF16)
    n = lc_moe_fp8_weights_size(shape)
    if n == 0:
        raise LcMoeError(2, "lc_moe_fp8_weights_size")
    out = torch.empty(n, dtype=torch.uint8, device=w_gate.device)
    lc_moe_quantize_weights(shape, w_gate, w_up, w_down, out)
    return out


def quantize_activations(x):
    """Block-FP8 form of bf16 rows x [rows, cols] (1 x 128 blocks): (codes uint8 [rows, cols],
    E8M0 scale bytes uint8 [rows, ceil(cols/128)])."""
    import torch
    rows, cols = x.shape
    if x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise TypeError("quantize_activations: x must be a contiguous bf16 tensor")
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, -(-cols // 128)), dtype=torch.uint8, device=x.device)
    lc_moe_quantize_activations(x, rows, cols, codes, scales)
    return codes, scales


def pack_weights(w_gate, w_up, w_down):
    """Packed form of bf16 expert weights (W_gate, W_up [N,I,d], W_down [N,d,I]) as a uint8
    device tensor, for ``forward(..., packed=...)`` / ``Weights.packed``."""
    import torch
    N, I, d = w_gate.shape
    shape = make_shape(1, d, N, 0, 1, I, BF16)
    n = lc_moe_packed_weights_size(shape)
    if n == 0:
        raise LcMoeError(2, "lc_moe_packed_weights_size")
    out = torch.empty(n, dtype=torch.uint8, device=w_gate.device)
    lc_moe_pack_weights(shape, w_gate, w_up, w_down, out)
    return out

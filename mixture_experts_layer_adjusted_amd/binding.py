"""Thin ctypes binding of libmoe.so (include/moe.h): argument marshalling only.

Every function has the name of the C entry point it calls, takes torch tensors
(device memory) where the C call takes device pointers, and raises MoeError on
a non-zero status.  Nothing here computes any part of the layer; if the
library has not been built the import of this module fails.
"""
from __future__ import annotations

import ctypes
import os

# torch must be loaded before libmoe.so: torch ships its own HIP runtime under
# the same soname (libamdhip64.so.7) as the ROCm one libmoe.so links, and only
# if torch's copy is already mapped does libmoe.so bind to it, leaving one HIP
# runtime in the process (two runtimes cannot share streams or device memory).
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_FP8_B128 = 0, 1, 2
MOE_FORWARD_EVENTS = 6
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down",
        "w_gate_scale", "w_up_scale", "w_down_scale", "sh_gate_scale", "sh_up_scale", "sh_down_scale")]


class WeightGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_SIG = {
    "moe_workspace_size": [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)],
    "moe_route": [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_route_noalloc": [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P],
    "moe_route_grouped": [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                          ctypes.c_size_t, _P],
    "moe_forward": [ctypes.POINTER(Shape), _P, ctypes.POINTER(Weights), _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_forward_profiled": [ctypes.POINTER(Shape), _P, ctypes.POINTER(Weights), _P, _P, _P, _P, ctypes.c_size_t,
                             _P, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32],
    "moe_update_bias": [ctypes.c_int32, ctypes.c_int64, _P, _P, ctypes.c_float, _P],
    "moe_prepare_weights": [ctypes.POINTER(Shape), ctypes.POINTER(Weights), _P, ctypes.POINTER(ctypes.c_size_t),
                            ctypes.POINTER(Weights), _P],
    "moe_quantize_weights": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P],
    "moe_quantize_act": [ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P],
    "moe_route_balance": [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P,
                          ctypes.c_size_t, _P],
    "moe_backward_workspace_size": [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)],
    "moe_backward": [ctypes.POINTER(Shape), _P, _P, ctypes.POINTER(Weights), _P, _P, _P, _P, _P,
                     ctypes.POINTER(WeightGrads), _P, ctypes.c_size_t, _P],
    "moe_saved_inputs_size": [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)],
    "moe_forward_train": [ctypes.POINTER(Shape), _P, ctypes.POINTER(Weights), _P, _P, _P, _P, ctypes.c_size_t, _P,
                          ctypes.c_size_t, _P],
    "moe_backward_saved": [ctypes.POINTER(Shape), _P, _P, ctypes.POINTER(Weights), _P, _P, _P, ctypes.c_size_t, _P,
                           _P, _P, ctypes.POINTER(WeightGrads), _P, ctypes.c_size_t, _P],
    "moe_status_string": [ctypes.c_int32],
}
for _name, _args in _SIG.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_char_p if _name == "moe_status_string" else ctypes.c_int


def exported_symbols():
    return list(_SIG)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise MoeError(fn, rc)


def make_shape(tokens, hidden, n_routed, top_k, n_shared, inter, dtype) -> Shape:
    return Shape(tokens, hidden, n_routed, top_k, n_shared, inter, dtype)


def make_weights(w_gate, w_up, w_down, sh_gate=None, sh_up=None, sh_down=None, scales=None) -> Weights:
    """scales: optional dict with keys w_gate_scale, ..., sh_down_scale (fp8 only)."""
    w = Weights(*(_ptr(t).value if t is not None else None
                  for t in (w_gate, w_up, w_down, sh_gate, sh_up, sh_down)))
    for k, t in (scales or {}).items():
        setattr(w, k, t.data_ptr() if t is not None else None)
    return w


def moe_route_balance(shape, seq_len, alpha, u, centroids, bias, topk_idx, topk_gate, expert_load, seq_loss,
                      workspace, stream=None):
    _check("moe_route_balance", _lib.moe_route_balance(
        ctypes.byref(shape), seq_len, ctypes.c_float(alpha), _ptr(u), _ptr(centroids), _ptr(bias), _ptr(topk_idx),
        _ptr(topk_gate), _ptr(expert_load), _ptr(seq_loss), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def make_weight_grads(w_gate, w_up, w_down, sh_gate=None, sh_up=None, sh_down=None) -> WeightGrads:
    return WeightGrads(*(_ptr(t).value if t is not None else None
                         for t in (w_gate, w_up, w_down, sh_gate, sh_up, sh_down)))


def moe_backward_workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_backward_workspace_size", _lib.moe_backward_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_backward(shape, u, centroids, weights, topk_idx, topk_gate, dout, du, d_centroids, weight_grads, workspace,
                 stream=None):
    _check("moe_backward", _lib.moe_backward(
        ctypes.byref(shape), _ptr(u), _ptr(centroids), ctypes.byref(weights), _ptr(topk_idx), _ptr(topk_gate),
        _ptr(dout), _ptr(du), _ptr(d_centroids), ctypes.byref(weight_grads), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def moe_saved_inputs_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_saved_inputs_size", _lib.moe_saved_inputs_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_forward_train(shape, u, weights: Weights, topk_idx, topk_gate, out, saved, workspace, stream=None):
    _check("moe_forward_train", _lib.moe_forward_train(
        ctypes.byref(shape), _ptr(u), ctypes.byref(weights), _ptr(topk_idx), _ptr(topk_gate), _ptr(out),
        _ptr(saved), _nbytes(saved), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_backward_saved(shape, u, centroids, weights, topk_idx, topk_gate, saved, dout, du, d_centroids,
                       weight_grads, workspace, stream=None):
    _check("moe_backward_saved", _lib.moe_backward_saved(
        ctypes.byref(shape), _ptr(u), _ptr(centroids), ctypes.byref(weights), _ptr(topk_idx), _ptr(topk_gate),
        _ptr(saved), _nbytes(saved), _ptr(dout), _ptr(du), _ptr(d_centroids), ctypes.byref(weight_grads),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", _lib.moe_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def moe_route(shape, u, centroids, bias, topk_idx, topk_gate, expert_load, workspace, stream=None):
    _check("moe_route", _lib.moe_route(ctypes.byref(shape), _ptr(u), _ptr(centroids), _ptr(bias), _ptr(topk_idx),
                                       _ptr(topk_gate), _ptr(expert_load), _ptr(workspace), _nbytes(workspace),
                                       _stream(stream)))


def moe_route_noalloc(shape, u, centroids, bias, topk_idx, topk_gate, expert_load, stream=None):
    _check("moe_route_noalloc", _lib.moe_route_noalloc(ctypes.byref(shape), _ptr(u), _ptr(centroids), _ptr(bias),
                                                       _ptr(topk_idx), _ptr(topk_gate), _ptr(expert_load),
                                                       _stream(stream)))


def moe_route_grouped(shape, n_groups, topk_groups, u, centroids, bias, topk_idx, topk_gate, expert_load, workspace,
                      stream=None):
    _check("moe_route_grouped", _lib.moe_route_grouped(
        ctypes.byref(shape), n_groups, topk_groups, _ptr(u), _ptr(centroids), _ptr(bias), _ptr(topk_idx),
        _ptr(topk_gate), _ptr(expert_load), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_forward(shape, u, weights: Weights, topk_idx, topk_gate, out, workspace, stream=None):
    _check("moe_forward", _lib.moe_forward(ctypes.byref(shape), _ptr(u), ctypes.byref(weights), _ptr(topk_idx),
                                           _ptr(topk_gate), _ptr(out), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_forward_profiled(shape, u, weights: Weights, topk_idx, topk_gate, out, workspace, events, stream=None):
    """events: MOE_FORWARD_EVENTS torch.cuda.Event(enable_timing=True) objects, recorded in order.

    torch creates an event's HIP handle on its first record(); record each event once
    beforehand so that a handle exists."""
    if any(not e.cuda_event for e in events):
        raise ValueError("moe_forward_profiled: an event has no HIP handle yet (record it once first)")
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check("moe_forward_profiled", _lib.moe_forward_profiled(
        ctypes.byref(shape), _ptr(u), ctypes.byref(weights), _ptr(topk_idx), _ptr(topk_gate), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream), arr, len(events)))


def moe_update_bias(n_routed, total_assignments, expert_load, bias, gamma, stream=None):
    _check("moe_update_bias", _lib.moe_update_bias(n_routed, total_assignments, _ptr(expert_load), _ptr(bias),
                                                   gamma, _stream(stream)))


def moe_prepare_weights(shape, logical, packed=None, stream=None, size_only=False):
    """size_only: returns the bytes `packed` needs.  Otherwise returns the prepared Weights (for
    FP8_B128 they point into `packed`, which must outlive them)."""
    n = ctypes.c_size_t(0 if packed is None else _nbytes(packed))
    if size_only:
        _check("moe_prepare_weights", _lib.moe_prepare_weights(ctypes.byref(shape), ctypes.byref(logical), None,
                                                               ctypes.byref(n), None, None))
        return n.value
    prepared = Weights()
    _check("moe_prepare_weights", _lib.moe_prepare_weights(ctypes.byref(shape), ctypes.byref(logical), _ptr(packed),
                                                           ctypes.byref(n), ctypes.byref(prepared), _stream(stream)))
    return prepared


def moe_quantize_weights(n_mats, rows, cols, w_bf16, codes, scales, stream=None):
    _check("moe_quantize_weights", _lib.moe_quantize_weights(n_mats, rows, cols, _ptr(w_bf16), _ptr(codes),
                                                             _ptr(scales), _stream(stream)))


def moe_quantize_act(rows, cols, x_bf16, codes, scales, stream=None):
    _check("moe_quantize_act", _lib.moe_quantize_act(rows, cols, _ptr(x_bf16), _ptr(codes), _ptr(scales),
                                                     _stream(stream)))


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def raw_lib():
    """The ctypes handle itself (for host-side error-path tests)."""
    return _lib

"""ctypes binding of liblatentmoe.so (C ABI in include/latentmoe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory and the stream.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblatentmoe.so")

LMOE_F32, LMOE_BF16 = 0, 1
ENTRY_ROUTE, ENTRY_DISPATCH, ENTRY_EXPERTS, ENTRY_FORWARD, ENTRY_ROUTED_BACKWARD, ENTRY_BACKWARD = 0, 1, 2, 3, 4, 5
STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "CAPACITY", 4: "WORKSPACE", 5: "HIP", 6: "RANGE"}

# every symbol include/latentmoe.h declares
EXPORTS = (
    "latentmoe_workspace_bytes", "latentmoe_status_string", "latentmoe_last_error",
    "latentmoe_route", "latentmoe_dispatch", "latentmoe_experts", "latentmoe_forward",
    "latentmoe_forward_timed", "latentmoe_route_softmax", "latentmoe_router_losses_workspace_bytes",
    "latentmoe_router_losses", "latentmoe_routed_backward", "latentmoe_backward", "latentmoe_forward_check",
    "latentmoe_forward_noalloc",
)
GRAD_NAMES = ("w_down", "w_router", "w_g", "w_u", "w_o", "sh_g", "sh_u", "sh_o", "rms_w", "w_up")
TIMING_EVENTS = 9
STEP_NAMES = ("latent_gemm", "router", "dispatch", "shared_gateup", "routed_gateup", "routed_down",
              "combine_rmsnorm", "merge_gemm")


class LatentMoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_latent", ctypes.c_int32),
        ("n_routed", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("ff_routed", ctypes.c_int32), ("ff_shared", ctypes.c_int32), ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
    ]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_NAMES]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_down", "w_router", "bias", "w_g", "w_u", "w_o", "sh_g", "sh_u", "sh_o", "rms_w", "w_up")]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, st, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    D = ctypes.POINTER(Dims)
    lib.latentmoe_workspace_bytes.argtypes = [D, i32]
    lib.latentmoe_workspace_bytes.restype = st
    lib.latentmoe_status_string.argtypes = [ctypes.c_int]
    lib.latentmoe_status_string.restype = ctypes.c_char_p
    lib.latentmoe_last_error.argtypes = []
    lib.latentmoe_last_error.restype = ctypes.c_char_p
    lib.latentmoe_route.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, st, vp]
    lib.latentmoe_dispatch.argtypes = [D, vp, vp, vp, vp, vp, vp, i64, ctypes.POINTER(i64), vp, st, vp]
    lib.latentmoe_experts.argtypes = [D, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, st, vp]
    lib.latentmoe_forward.argtypes = [D, ctypes.POINTER(Weights), vp, vp, vp, vp, vp,
                                      ctypes.POINTER(i64), vp, st, vp]
    lib.latentmoe_forward_timed.argtypes = [D, ctypes.POINTER(Weights), vp, vp, vp, vp, vp, vp, st, vp,
                                            ctypes.POINTER(vp), i32]
    lib.latentmoe_route_softmax.argtypes = [D, vp, vp, vp, vp, vp, vp, st, vp]
    lib.latentmoe_forward_check.argtypes = [D, vp, st, vp]
    lib.latentmoe_forward_noalloc.argtypes = [D, ctypes.POINTER(Weights), vp, vp, vp, vp, vp, vp]
    lib.latentmoe_router_losses_workspace_bytes.argtypes = [D]
    lib.latentmoe_router_losses_workspace_bytes.restype = st
    lib.latentmoe_router_losses.argtypes = [D, vp, vp, vp, vp, st, vp]
    lib.latentmoe_routed_backward.argtypes = [D] + [vp] * 13 + [st, vp]
    lib.latentmoe_backward.argtypes = [D, ctypes.POINTER(Weights), vp, vp, vp, vp, vp, ctypes.POINTER(Grads), vp,
                                       st, vp]
    for fn in ("latentmoe_route", "latentmoe_dispatch", "latentmoe_experts", "latentmoe_forward",
               "latentmoe_forward_timed", "latentmoe_route_softmax", "latentmoe_router_losses",
               "latentmoe_routed_backward", "latentmoe_backward", "latentmoe_forward_check",
               "latentmoe_forward_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int):
    if status != 0:
        raise LatentMoEError(status, load().latentmoe_last_error().decode())


def ptr(t) -> int | None:
    """Device (or host) address of a tensor, None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None, device=None) -> int | None:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def make_dims(n_tokens, d_model, d_latent, n_routed, top_k, n_shared, ff_routed, ff_shared,
              dtype="bf16", beta1=4.0, beta2=25.0, rms_eps=1e-6) -> Dims:
    return Dims(n_tokens, d_model, d_latent, n_routed, top_k, n_shared, ff_routed, ff_shared,
                beta1, beta2, rms_eps, LMOE_BF16 if dtype == "bf16" else LMOE_F32)


def dims_of(cfg, n_tokens=None) -> Dims:
    """Dims of a layer configuration object (fields named as in lmoe_dims)."""
    return make_dims(cfg.n_tokens if n_tokens is None else n_tokens, cfg.d_model, cfg.d_latent,
                     cfg.n_routed, cfg.top_k, cfg.n_shared, cfg.ff_routed, cfg.ff_shared, cfg.dtype,
                     cfg.beta1, cfg.beta2, cfg.rms_eps)


def workspace_bytes(dims: Dims, entry: int) -> int:
    return int(load().latentmoe_workspace_bytes(ctypes.byref(dims), entry))


# ------------------------------------------------------------- entry points
def latentmoe_route(dims, x, w_router, bias, ids, probs, logits=None, workspace=None, stream=None):
    ws = workspace
    check(load().latentmoe_route(ctypes.byref(dims), ptr(x), ptr(w_router), ptr(bias), ptr(ids),
                                 ptr(probs), ptr(logits), ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                 stream_handle(stream)))


def latentmoe_route_softmax(dims, x, w_router, ids, probs, logits=None, workspace=None, stream=None):
    ws = workspace
    check(load().latentmoe_route_softmax(ctypes.byref(dims), ptr(x), ptr(w_router), ptr(ids), ptr(probs),
                                         ptr(logits), ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(),
                                         stream_handle(stream)))


def router_losses_workspace_bytes(dims: Dims) -> int:
    return int(load().latentmoe_router_losses_workspace_bytes(ctypes.byref(dims)))


def latentmoe_router_losses(dims, logits, counts, out, workspace=None, stream=None):
    ws = workspace
    check(load().latentmoe_router_losses(ctypes.byref(dims), ptr(logits), ptr(counts), ptr(out), ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(),
                                         stream_handle(stream)))


def latentmoe_routed_backward(dims, z, ids, probs, w_g, w_u, w_o, du, dz, dprobs, dw_g, dw_u, dw_o,
                              workspace=None, stream=None):
    ws = workspace
    check(load().latentmoe_routed_backward(ctypes.byref(dims), ptr(z), ptr(ids), ptr(probs), ptr(w_g), ptr(w_u),
                                           ptr(w_o), ptr(du), ptr(dz), ptr(dprobs), ptr(dw_g), ptr(dw_u),
                                           ptr(dw_o), ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                           stream_handle(stream)))


def latentmoe_backward(dims, weights, x, ids, probs, dy, dx, grads: dict, workspace=None, stream=None):
    """grads: dict of output tensors keyed by GRAD_NAMES (sh_* may be absent when n_s = 0)."""
    W = weights if isinstance(weights, Weights) else weights_struct(weights)
    G = Grads(*[ptr(grads.get(n)) for n in GRAD_NAMES])
    ws = workspace
    check(load().latentmoe_backward(ctypes.byref(dims), ctypes.byref(W), ptr(x), ptr(ids), ptr(probs), ptr(dy),
                                    ptr(dx), ctypes.byref(G), ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(), stream_handle(stream)))


def latentmoe_dispatch(dims, ids, z, counts, offsets, order, padded=None, capacity=0,
                       workspace=None, stream=None) -> int:
    C = ctypes.c_int64(0)
    ws = workspace
    status = load().latentmoe_dispatch(ctypes.byref(dims), ptr(ids), ptr(z), ptr(counts), ptr(offsets),
                                       ptr(order), ptr(padded), int(capacity), ctypes.byref(C), ptr(ws),
                                       0 if ws is None else ws.numel() * ws.element_size(),
                                       stream_handle(stream))
    if status == 3:
        raise LatentMoEError(3, load().latentmoe_last_error().decode() + f" (C={C.value})")
    check(status)
    return C.value


def latentmoe_experts(dims, padded, C, counts, offsets, order, probs, w_g, w_u, w_o, u,
                      workspace=None, stream=None):
    ws = workspace
    check(load().latentmoe_experts(ctypes.byref(dims), ptr(padded), int(C), ptr(counts), ptr(offsets),
                                   ptr(order), ptr(probs), ptr(w_g), ptr(w_u), ptr(w_o), ptr(u), ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   stream_handle(stream)))


def weights_struct(w: dict) -> Weights:
    return Weights(*[ptr(w.get(n)) for n in (
        "w_down", "w_router", "bias", "w_g", "w_u", "w_o", "sh_g", "sh_u", "sh_o", "rms_w", "w_up")])


def latentmoe_forward(dims, weights, x, y, ids, probs, counts, want_capacity=True, workspace=None,
                      stream=None) -> int | None:
    """weights: dict of tensors keyed like lmoe_weights, or a prepared Weights struct."""
    W = weights if isinstance(weights, Weights) else weights_struct(weights)
    C = ctypes.c_int64(0)
    ws = workspace
    check(load().latentmoe_forward(ctypes.byref(dims), ctypes.byref(W), ptr(x), ptr(y), ptr(ids), ptr(probs),
                                   ptr(counts), ctypes.byref(C) if want_capacity else None, ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   stream_handle(stream)))
    return C.value if want_capacity else None


def latentmoe_forward_timed(dims, weights, x, y, ids, probs, counts, events, workspace=None, stream=None):
    """events: TIMING_EVENTS torch.cuda.Event(enable_timing=True) objects; after the
    call events[i-1].elapsed_time(events[i]) is step i's time (STEP_NAMES)."""
    W = weights if isinstance(weights, Weights) else weights_struct(weights)
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    ws = workspace
    check(load().latentmoe_forward_timed(ctypes.byref(dims), ctypes.byref(W), ptr(x), ptr(y), ptr(ids),
                                         ptr(probs), ptr(counts), ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(),
                                         stream_handle(stream), handles, len(events)))


def latentmoe_forward_noalloc(dims, weights, x, y, ids, probs, counts, stream=None):
    """latentmoe_forward without a workspace (the library's fixed device
    scratch; asynchronous, no capacity read-back)."""
    W = weights if isinstance(weights, Weights) else weights_struct(weights)
    check(load().latentmoe_forward_noalloc(ctypes.byref(dims), ctypes.byref(W), ptr(x), ptr(y), ptr(ids),
                                           ptr(probs), ptr(counts), stream_handle(stream)))


def latentmoe_forward_check(dims, workspace, stream=None):
    """Raises LatentMoEError (status RANGE) if the last forward enqueued with
    this workspace (None: the fixed scratch of latentmoe_forward_noalloc)
    left fp16's range in an intermediate."""
    ws = workspace
    check(load().latentmoe_forward_check(ctypes.byref(dims), ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(),
                                         stream_handle(stream)))

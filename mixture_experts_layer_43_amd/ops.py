"""Torch-tensor wrappers over the libmoe C ABI (names follow include/moe.h).

PyTorch only supplies device memory and the current HIP stream; every step
of the layer runs in the library's kernels.  Each wrapper checks shapes,
dtypes and devices of its tensors (the C ABI sees raw pointers), allocates
its outputs and workspace with torch.empty, and enqueues on
torch.cuda.current_stream().
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import MoeLayer, call

_DT = {"f32": (_lib.MOE_F32, torch.float32), "bf16": (_lib.MOE_BF16, torch.bfloat16)}
_GATE = {"softmax_topk": _lib.MOE_GATE_SOFTMAX_TOPK, "topk_softmax": _lib.MOE_GATE_TOPK_SOFTMAX}
_FFN = {"silu": _lib.MOE_FFN_SILU_GATED, "relu": _lib.MOE_FFN_RELU}
_BIAS = {"logits": _lib.MOE_BIAS_LOGITS, "selection": _lib.MOE_BIAS_SELECTION}
_LAYOUT = {"row_major": _lib.MOE_WEIGHTS_ROW_MAJOR, "packed": _lib.MOE_WEIGHTS_PACKED}
_RLAYOUT = {"row_major": _lib.MOE_ROUTER_ROW_MAJOR, "packed": _lib.MOE_ROUTER_PACKED}


@dataclass(frozen=True)
class Layer:
    """Shape of one MoE layer: N_r routed experts of width I, K_s shared experts
    of width I_s, top-K' routing."""
    d_model: int
    n_routed: int
    n_shared: int
    top_k: int
    d_ff: int
    d_ff_shared: int
    gate: str = "softmax_topk"
    dtype: str = "bf16"
    capacity: int = 0       # slots per expert per token group; 0 = dropless
    group_size: int = 0     # tokens per capacity group; 0 = the whole batch
    ffn: str = "silu"       # "silu" (W1, W3, W2) or "relu" (wi = w_gate, wo = w_down)
    bias_mode: str = "logits"  # "logits": bias in selection and gates; "selection": selection only
    weight_layout: str = "row_major"  # or "packed" (weights converted by pack_weights)
    router_layout: str = "row_major"  # or "packed" (w_router converted by pack_router)

    @classmethod
    def of(cls, cfg) -> "Layer":
        return cls(cfg.d_model, cfg.n_routed, cfg.n_shared, cfg.top_k, cfg.d_ff,
                   cfg.d_ff_shared, cfg.gate, cfg.dtype, getattr(cfg, "capacity", 0),
                   getattr(cfg, "group_size", 0), getattr(cfg, "ffn", "silu"),
                   getattr(cfg, "bias_mode", "logits"), getattr(cfg, "weight_layout", "row_major"),
                   getattr(cfg, "router_layout", "row_major"))

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DT[self.dtype][1]

    def c(self) -> MoeLayer:
        return MoeLayer(self.d_model, self.n_routed, self.n_shared, self.top_k, self.d_ff,
                        self.d_ff_shared, _GATE[self.gate], _DT[self.dtype][0], self.capacity,
                        self.group_size, _FFN[self.ffn], _BIAS[self.bias_mode],
                        _LAYOUT[self.weight_layout], _RLAYOUT[self.router_layout])

    @property
    def router_shape(self) -> tuple:
        """Shape of w_router: [N_r, d], or [MOE_ROUTER_PAD_ROWS(N_r), d] packed."""
        if self.router_layout == "packed":
            return (_lib.router_pad_rows(self.n_routed), self.d_model)
        return (self.n_routed, self.d_model)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t, shape, dtype, name, device=None):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def workspace_size(layer: Layer, T: int) -> int:
    n = ctypes.c_size_t(0)
    call("moe_workspace_size", ctypes.byref(layer.c()), T, ctypes.byref(n))
    return n.value


def workspace(layer: Layer, T: int, device) -> torch.Tensor:
    return torch.empty(max(workspace_size(layer, T), 1), dtype=torch.uint8, device=device)


def route(layer: Layer, x, w_router, bias=None):
    T = x.shape[0]
    dt = layer.torch_dtype
    _check(x, (T, layer.d_model), dt, "x")
    _check(w_router, layer.router_shape, torch.float32, "w_router", x.device)
    _check(bias, (layer.n_routed,), torch.float32, "bias", x.device)
    idx = torch.empty((T, layer.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, layer.top_k), dtype=torch.float32, device=x.device)
    call("moe_route", ctypes.byref(layer.c()), T, _p(x), _p(w_router), _p(bias), _p(idx), _p(w),
         _stream())
    return idx, w


def route_noisy(layer: Layer, x, w_router, bias, w_noise, noise):
    """Noisy top-k gating: the logits gain noise * softplus(x w_noise^T)."""
    T = x.shape[0]
    dt = layer.torch_dtype
    _check(x, (T, layer.d_model), dt, "x")
    _check(w_router, (layer.n_routed, layer.d_model), torch.float32, "w_router", x.device)
    _check(bias, (layer.n_routed,), torch.float32, "bias", x.device)
    _check(w_noise, (layer.n_routed, layer.d_model), torch.float32, "w_noise", x.device)
    _check(noise, (T, layer.n_routed), torch.float32, "noise", x.device)
    idx = torch.empty((T, layer.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, layer.top_k), dtype=torch.float32, device=x.device)
    call("moe_route_noisy", ctypes.byref(layer.c()), T, _p(x), _p(w_router), _p(bias), _p(w_noise),
         _p(noise), _p(idx), _p(w), _stream())
    return idx, w


def pack_router(layer: Layer, w_router):
    """w_router [N_r, d] fp32 in the packed router order: [MOE_ROUTER_PAD_ROWS(N_r), d]."""
    _check(w_router, (layer.n_routed, layer.d_model), torch.float32, "w_router")
    out = torch.empty((_lib.router_pad_rows(layer.n_routed), layer.d_model), dtype=torch.float32,
                      device=w_router.device)
    call("moe_pack_router", ctypes.byref(layer.c()), _p(w_router), _p(out), _stream())
    return out


def pack_weights(layer: Layer, w):
    """The packed copy of a [count, rows, cols] (or [rows, cols]) bf16 weight tensor."""
    if w is None:
        return None
    if w.dtype != torch.bfloat16 or not w.is_cuda or not w.is_contiguous() or w.dim() not in (2, 3):
        raise ValueError("pack_weights: need a contiguous bf16 GPU tensor of rank 2 or 3")
    count, rows, cols = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
    out = torch.empty_like(w)
    call("moe_pack_weights", ctypes.byref(layer.c()), count, rows, cols, _p(w), _p(out), _stream())
    return out


def stats_len(layer: Layer, n_devices: int) -> int:
    return 2 * layer.n_routed + 2 * n_devices + 3


def split_stats(layer: Layer, n_devices: int, stats) -> dict:
    """Name the parts of a moe_route_stats output vector (include/moe.h)."""
    n, D = layer.n_routed, n_devices
    return {"P": stats[:n], "f": stats[n:2 * n], "f_dev": stats[2 * n:2 * n + D],
            "P_dev": stats[2 * n + D:2 * n + 2 * D], "l_exp": stats[2 * n + 2 * D],
            "l_dev": stats[2 * n + 2 * D + 1], "z_loss": stats[2 * n + 2 * D + 2]}


def route_stats(layer: Layer, x, w_router, bias=None, n_devices: int = 1, lse: bool = False,
                ws=None):
    """Router plus routing statistics: (topk_idx, topk_w, stats [2N+2D+3], lse [T] or None)."""
    T = x.shape[0]
    dt = layer.torch_dtype
    _check(x, (T, layer.d_model), dt, "x")
    _check(w_router, layer.router_shape, torch.float32, "w_router", x.device)
    _check(bias, (layer.n_routed,), torch.float32, "bias", x.device)
    idx = torch.empty((T, layer.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, layer.top_k), dtype=torch.float32, device=x.device)
    stats = torch.empty(stats_len(layer, n_devices), dtype=torch.float32, device=x.device)
    l = torch.empty(T, dtype=torch.float32, device=x.device) if lse else None
    ws = workspace(layer, T, x.device) if ws is None else ws
    call("moe_route_stats", ctypes.byref(layer.c()), T, _p(x), _p(w_router), _p(bias), n_devices,
         _p(idx), _p(w), _p(stats), _p(l), _p(ws), ws.numel(), _stream())
    return idx, w, stats, l


def permute(layer: Layer, topk_idx, x=None, ws=None):
    """Dispatch.  x given: also returns x_perm (rows of x in dispatch order)."""
    T = topk_idx.shape[0]
    dev = topk_idx.device
    _check(topk_idx, (T, layer.top_k), torch.int32, "topk_idx")
    _check(x, (T, layer.d_model), layer.torch_dtype, "x", dev)
    P = T * layer.top_k
    out = {
        "counts": torch.empty(layer.n_routed, dtype=torch.int32, device=dev),
        "offsets": torch.empty(layer.n_routed + 1, dtype=torch.int32, device=dev),
        "row_token": torch.empty(P, dtype=torch.int32, device=dev),
        "slot_row": torch.empty(P, dtype=torch.int32, device=dev),
        "x_perm": None if x is None else torch.empty((P, layer.d_model), dtype=x.dtype, device=dev),
    }
    ws = workspace(layer, T, dev) if ws is None else ws
    call("moe_permute", ctypes.byref(layer.c()), T, _p(topk_idx), _p(x), _p(out["counts"]),
         _p(out["offsets"]), _p(out["row_token"]), _p(out["slot_row"]), _p(out["x_perm"]),
         _p(ws), ws.numel(), _stream())
    return out


def expert_ffn(layer: Layer, T: int, offsets, x_perm, w_gate, w_up, w_down, ws=None):
    dt, dev = layer.torch_dtype, x_perm.device
    P, d, I, N = T * layer.top_k, layer.d_model, layer.d_ff, layer.n_routed
    _check(offsets, (N + 1,), torch.int32, "offsets", dev)
    _check(x_perm, (P, d), dt, "x_perm")
    _check(w_gate, (N, I, d), dt, "w_gate", dev)
    _check(w_up, (N, I, d), dt, "w_up", dev)
    _check(w_down, (N, d, I), dt, "w_down", dev)
    y_perm = torch.empty((P, d), dtype=dt, device=dev)
    ws = workspace(layer, T, dev) if ws is None else ws
    call("moe_expert_ffn", ctypes.byref(layer.c()), T, _p(offsets), _p(x_perm), _p(w_gate),
         _p(w_up), _p(w_down), _p(y_perm), _p(ws), ws.numel(), _stream())
    return y_perm


def shared_ffn(layer: Layer, x, ws_gate, ws_up, ws_down, ws=None):
    T = x.shape[0]
    dt, dev = layer.torch_dtype, x.device
    d, Ks, Is = layer.d_model, layer.n_shared, layer.d_ff_shared
    _check(x, (T, d), dt, "x")
    if Ks > 0:
        _check(ws_gate, (Ks, Is, d), dt, "ws_gate", dev)
        _check(ws_up, (Ks, Is, d), dt, "ws_up", dev)
        _check(ws_down, (Ks, d, Is), dt, "ws_down", dev)
    y = torch.empty((T, d), dtype=dt, device=dev)
    ws = workspace(layer, T, dev) if ws is None else ws
    call("moe_shared_ffn", ctypes.byref(layer.c()), T, _p(x), _p(ws_gate), _p(ws_up),
         _p(ws_down), _p(y), _p(ws), ws.numel(), _stream())
    return y


def combine(layer: Layer, y_perm, slot_row, topk_w, y_shared=None, residual=None):
    T = topk_w.shape[0]
    dt, dev = layer.torch_dtype, y_perm.device
    P, d = T * layer.top_k, layer.d_model
    _check(y_perm, (P, d), dt, "y_perm")
    _check(slot_row, (P,), torch.int32, "slot_row", dev)
    _check(topk_w, (T, layer.top_k), torch.float32, "topk_w", dev)
    _check(y_shared, (T, d), dt, "y_shared", dev)
    _check(residual, (T, d), dt, "residual", dev)
    y = torch.empty((T, d), dtype=dt, device=dev)
    call("moe_combine", ctypes.byref(layer.c()), T, _p(y_perm), _p(slot_row), _p(topk_w),
         _p(y_shared), _p(residual), _p(y), _stream())
    return y


class Forward:
    """The whole layer with preallocated outputs and workspace (repeat calls allocate nothing).

    noalloc=True calls moe_forward_noalloc instead: no workspace tensor, the
    scratch comes from the library's static device array (include/moe.h)."""

    def __init__(self, layer: Layer, T: int, device, noalloc: bool = False):
        device = torch.device(device)
        if device.type == "cuda" and device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.layer, self.T, self.device, self.noalloc = layer, T, device, noalloc
        self._c = layer.c()
        self.ws = None if noalloc else workspace(layer, T, device)
        self.y = torch.empty((T, layer.d_model), dtype=layer.torch_dtype, device=device)
        self.topk_idx = torch.empty((T, layer.top_k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, layer.top_k), dtype=torch.float32, device=device)
        self.counts = torch.empty(layer.n_routed, dtype=torch.int32, device=device)
        self.offsets = torch.empty(layer.n_routed + 1, dtype=torch.int32, device=device)

    def check(self, x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, residual):
        L, dt, dev = self.layer, self.layer.torch_dtype, self.device
        d, N, I, Ks, Is = L.d_model, L.n_routed, L.d_ff, L.n_shared, L.d_ff_shared
        _check(x, (self.T, d), dt, "x", dev)
        _check(w_router, self.layer.router_shape, torch.float32, "w_router", dev)
        _check(bias, (N,), torch.float32, "bias", dev)
        _check(w_gate, (N, I, d), dt, "w_gate", dev)
        _check(w_up, (N, I, d), dt, "w_up", dev)
        _check(w_down, (N, d, I), dt, "w_down", dev)
        if Ks > 0:
            _check(ws_gate, (Ks, Is, d), dt, "ws_gate", dev)
            _check(ws_up, (Ks, Is, d), dt, "ws_up", dev)
            _check(ws_down, (Ks, d, Is), dt, "ws_down", dev)
        _check(residual, (self.T, d), dt, "residual", dev)

    def __call__(self, x, w_router, bias, w_gate, w_up, w_down, ws_gate=None, ws_up=None,
                 ws_down=None, residual=None, checked=False):
        if not checked:
            self.check(x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, residual)
        if self.noalloc:
            call("moe_forward_noalloc", ctypes.byref(self._c), self.T, _p(x), _p(w_router), _p(bias),
                 _p(w_gate), _p(w_up), _p(w_down), _p(ws_gate), _p(ws_up), _p(ws_down),
                 _p(residual), _p(self.y), _p(self.topk_idx), _p(self.topk_w), _p(self.counts),
                 _p(self.offsets), _stream())
            return self.y
        call("moe_forward", ctypes.byref(self._c), self.T, _p(x), _p(w_router), _p(bias),
             _p(w_gate), _p(w_up), _p(w_down), _p(ws_gate), _p(ws_up), _p(ws_down), _p(residual),
             _p(self.y), _p(self.topk_idx), _p(self.topk_w), _p(self.counts), _p(self.offsets),
             _p(self.ws), self.ws.numel(), _stream())
        return self.y


def forward(layer: Layer, x, w_router, bias, w_gate, w_up, w_down, ws_gate=None, ws_up=None,
            ws_down=None, residual=None):
    f = Forward(layer, x.shape[0], x.device)
    y = f(x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, residual)
    return {"y": y, "topk_idx": f.topk_idx, "topk_w": f.topk_w, "counts": f.counts,
            "offsets": f.offsets}

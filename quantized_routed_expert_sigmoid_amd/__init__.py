"""Python binding of libcolibri (include/colibri.h): one sigmoid-routed,
quantised mixture-of-experts layer forward on an MI355X (gfx950).

Argument marshalling only.  Every step of the layer runs in the library's
HIP kernels; PyTorch provides device memory and the current stream.  The
library is built in-tree by ``python -m quantized_routed_expert_sigmoid_amd.build``;
importing works without it, but every call that needs it raises if it is
missing -- there is no other implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcolibri.so")

COLI_OK, COLI_E_INVAL, COLI_E_UNSUPPORTED, COLI_E_WORKSPACE, COLI_E_HIP = 0, 1, 2, 3, 4
COLI_Q8, COLI_Q4, COLI_Q2 = 8, 4, 2
COLI_N_STAGE_EVENTS = 6
STAGES = ("route", "dispatch", "gate_up", "down", "combine")

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class QBankDesc(ctypes.Structure):
    """coli_qbank"""
    _fields_ = [("data", _vp), ("row_scale", _vp), ("n_mat", _i32), ("rows", _i32), ("K", _i32),
                ("qtype", _i32)]


class LayerDesc(ctypes.Structure):
    """coli_moe_layer"""
    _fields_ = [("hidden", _i32), ("inter", _i32), ("n_experts", _i32), ("top_k", _i32),
                ("routed_scaling_factor", ctypes.c_float), ("router_w", _vp), ("router_bias", _vp),
                ("gate", QBankDesc), ("up", QBankDesc), ("down", QBankDesc), ("has_shared", _i32),
                ("sh_gate", QBankDesc), ("sh_up", QBankDesc), ("sh_down", QBankDesc),
                ("n_group", _i32), ("topk_group", _i32), ("top_p", ctypes.c_float)]


class ColibriError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_routed_expert_sigmoid_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.colibri_status_string.restype = ctypes.c_char_p
        L.colibri_status_string.argtypes = [ctypes.c_int]
        L.colibri_workspace_bytes.restype = ctypes.c_size_t
        L.colibri_workspace_bytes.argtypes = [_vp, _i32]
        L.colibri_expert_ffn_workspace_bytes.restype = ctypes.c_size_t
        L.colibri_expert_ffn_workspace_bytes.argtypes = [_vp, _vp, _i32, _i32]
        L.colibri_quantize_q8_0.restype = ctypes.c_int
        L.colibri_quantize_q8_0.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp]
        L.colibri_route.restype = ctypes.c_int
        L.colibri_route.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.colibri_moe_dispatch.restype = ctypes.c_int
        L.colibri_moe_dispatch.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                           ctypes.c_size_t, _vp]
        L.colibri_expert_ffn_q.restype = ctypes.c_int
        L.colibri_expert_ffn_q.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp,
                                           ctypes.c_size_t, _vp]
        L.colibri_moe_layer_forward.restype = ctypes.c_int
        L.colibri_moe_layer_forward.argtypes = [_vp, _vp, _i32, _vp, _vp, ctypes.c_size_t, _vp]
        L.colibri_moe_layer_forward_staged.restype = ctypes.c_int
        L.colibri_moe_layer_forward_staged.argtypes = [_vp, _vp, _i32, _vp, _vp, ctypes.c_size_t, _vp,
                                                       _vp]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().colibri_status_string(status).decode()


def _check(status: int, what: str):
    if status != COLI_OK:
        raise ColibriError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------

@dataclass
class QBank:
    """n_mat quantised matrices [rows][K]: data uint8 [n_mat][rows][K*qtype/8],
    row scales fp32 [n_mat][rows] (device tensors)."""
    data: torch.Tensor
    scale: torch.Tensor
    qtype: int

    def desc(self) -> QBankDesc:
        n_mat, rows, rb = self.data.shape
        return QBankDesc(_ptr(self.data), _ptr(self.scale), n_mat, rows, rb * 8 // self.qtype,
                         self.qtype)


class MoELayer:
    """Device tensors of one layer plus its C descriptor."""

    def __init__(self, hidden: int, inter: int, n_experts: int, top_k: int, rsf: float,
                 router_w: torch.Tensor, router_bias: torch.Tensor, gate: QBank, up: QBank,
                 down: QBank, shared: Optional[Sequence[QBank]] = None,
                 n_group: int = 1, topk_group: int = 1, top_p: float = 1.0):
        self.hidden, self.inter, self.n_experts, self.top_k, self.rsf = hidden, inter, n_experts, top_k, rsf
        self.router_w, self.router_bias = router_w, router_bias
        self.gate, self.up, self.down = gate, up, down
        self.shared = tuple(shared) if shared else None
        sh = self.shared or (gate, up, down)
        self.desc = LayerDesc(hidden, inter, n_experts, top_k, rsf, _ptr(router_w), _ptr(router_bias),
                              gate.desc(), up.desc(), down.desc(), 1 if self.shared else 0,
                              sh[0].desc(), sh[1].desc(), sh[2].desc(), n_group, topk_group, top_p)

    def workspace_bytes(self, S: int) -> int:
        n = lib().colibri_workspace_bytes(ctypes.byref(self.desc), S)
        if n == 0:
            raise ColibriError(COLI_E_INVAL, "colibri_workspace_bytes")
        return n

    def workspace(self, S: int) -> torch.Tensor:
        return torch.empty(self.workspace_bytes(S), dtype=torch.uint8, device="cuda")


def quantize_q8_0(x: torch.Tensor):
    """x fp32 [rows][K] -> (codes int8 [rows][K], scales fp32 [rows][K/32])."""
    rows, K = x.shape
    q = torch.empty(rows, K, dtype=torch.int8, device=x.device)
    d = torch.empty(rows, K // 32, dtype=torch.float32, device=x.device)
    _check(lib().colibri_quantize_q8_0(_ptr(x), rows, K, _ptr(q), _ptr(d), _stream()),
           "colibri_quantize_q8_0")
    return q, d


def route(layer: MoELayer, x: torch.Tensor, ws: Optional[torch.Tensor] = None):
    """-> (ids int32 [S][k], weights fp32 [S][k])."""
    S = x.shape[0]
    ws = layer.workspace(S) if ws is None else ws
    ids = torch.empty(S, layer.top_k, dtype=torch.int32, device=x.device)
    w = torch.empty(S, layer.top_k, dtype=torch.float32, device=x.device)
    _check(lib().colibri_route(ctypes.byref(layer.desc), _ptr(x), S, _ptr(ids), _ptr(w), _ptr(ws),
                               ws.numel(), _stream()), "colibri_route")
    return ids, w


def moe_dispatch(ids: torch.Tensor, n_experts: int):
    """ids int32 [S][k] -> (offsets [E+1], sorted [S*k], active [E], n_active [1])."""
    S, k = ids.shape
    dev = ids.device
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    srt = torch.empty(max(S * k, 1), dtype=torch.int32, device=dev)
    active = torch.full((n_experts,), -1, dtype=torch.int32, device=dev)
    n_active = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().colibri_moe_dispatch(_ptr(ids), S, k, n_experts, _ptr(offsets), _ptr(srt),
                                      _ptr(active), _ptr(n_active), None, 0, _stream()),
           "colibri_moe_dispatch")
    return offsets, srt[:S * k], active, n_active


def expert_ffn_q(gate: QBank, up: QBank, down: QBank, xq: torch.Tensor, xd: torch.Tensor,
                 offsets: torch.Tensor, sorted_pairs: torch.Tensor, k: int):
    """-> y fp32 [S*k][hidden] in sorted order."""
    S, H = xq.shape
    g, u, d = gate.desc(), up.desc(), down.desc()
    y = torch.empty(S * k, H, dtype=torch.float32, device=xq.device)
    n = lib().colibri_expert_ffn_workspace_bytes(ctypes.byref(g), ctypes.byref(d), S, k)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=xq.device)
    _check(lib().colibri_expert_ffn_q(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), _ptr(xq),
                                      _ptr(xd), S, _ptr(offsets), _ptr(sorted_pairs), k, _ptr(y),
                                      _ptr(ws), ws.numel(), _stream()), "colibri_expert_ffn_q")
    return y


def moe_layer_forward(layer: MoELayer, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out fp32 [S][hidden] = the layer applied to x fp32 [S][hidden]."""
    S = x.shape[0]
    out = torch.empty_like(x) if out is None else out
    ws = layer.workspace(S) if ws is None else ws
    _check(lib().colibri_moe_layer_forward(ctypes.byref(layer.desc), _ptr(x), S, _ptr(out), _ptr(ws),
                                           ws.numel(), _stream()), "colibri_moe_layer_forward")
    return out


def moe_layer_forward_staged(layer: MoELayer, x: torch.Tensor, out: torch.Tensor, ws: torch.Tensor,
                             events) -> torch.Tensor:
    """The layer forward recording COLI_N_STAGE_EVENTS caller-created hipEvent_t
    handles (integers) between its stages on the current stream."""
    arr = (ctypes.c_void_p * COLI_N_STAGE_EVENTS)(*events)
    _check(lib().colibri_moe_layer_forward_staged(ctypes.byref(layer.desc), _ptr(x), x.shape[0],
                                                  _ptr(out), _ptr(ws), ws.numel(), _stream(), arr),
           "colibri_moe_layer_forward_staged")
    return out

"""Python binding of libcolibri (include/colibri.h): one sigmoid-routed,
quantised mixture-of-experts layer forward on an MI355X (gfx950).

Argument marshalling only.  Every step of the layer runs in the library's
HIP kernels; PyTorch provides device memory and the current stream.  The
library is built in-tree by ``python -m quantized_routed_expert_sigmoid_amd.build``;
importing works without it, but every call that needs it raises if it is
missing -- there is no other implementation to fall back to.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcolibri.so")
# the test-only build (include/colibri_debug.h): the same kernels, which also
# dump the block partials of one requested slice
DEBUG_LIB_PATH = os.path.join(PKG, "libcolibri_debug.so")

COLI_OK, COLI_E_INVAL, COLI_E_UNSUPPORTED, COLI_E_WORKSPACE, COLI_E_HIP, COLI_E_SCRATCH = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 16 << 20  # COLI_NOALLOC_SCRATCH_BYTES
COLI_Q8, COLI_Q4, COLI_Q2 = 8, 4, 2
COLI_N_STAGE_EVENTS = 6
STAGES = ("route", "dispatch", "gate_up", "down", "combine")

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class QBankDesc(ctypes.Structure):
    """coli_qbank"""
    _fields_ = [("data", _vp), ("row_scale", _vp), ("n_mat", _i32), ("rows", _i32), ("K", _i32),
                ("qtype", _i32), ("group", _i32)]


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
        _lib = _load(LIB_PATH)
    return _lib


def _load(path: str):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m quantized_routed_expert_sigmoid_amd.build`")
    L = ctypes.CDLL(path)
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
    L.colibri_moe_layer_forward_noalloc.restype = ctypes.c_int
    L.colibri_moe_layer_forward_noalloc.argtypes = [_vp, _vp, _i32, _vp, _vp]
    L.colibri_moe_layer_forward_staged.restype = ctypes.c_int
    L.colibri_moe_layer_forward_staged.argtypes = [_vp, _vp, _i32, _vp, _vp, ctypes.c_size_t, _vp,
                                                   _vp]
    for name, res, args in [
            ("colibri_cache_create", ctypes.c_int, [_i32, _i32, ctypes.POINTER(_vp)]),
            ("colibri_cache_destroy", None, [_vp]),
            ("colibri_cache_pin", ctypes.c_int, [_vp, _vp, _i32, _vp, _vp]),
            ("colibri_cache_unpin", None, [_vp]),
            ("colibri_cache_plan", ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _vp]),
            ("colibri_cache_prefetch", ctypes.c_int, [_vp, _vp, _i32, _vp, _vp]),
            ("colibri_tier_prefetch", ctypes.c_int, [_vp, _vp, _i32, _vp]),
            ("colibri_cache_stats", ctypes.c_int, [_vp, _vp]),
            ("colibri_cache_state", ctypes.c_int, [_vp, _vp, _vp]),
            ("colibri_tier_slot_bytes", ctypes.c_size_t, [_vp, _i32]),
            ("colibri_tier_create", ctypes.c_int, [_vp, _i32, _vp, ctypes.c_size_t,
                                                   ctypes.POINTER(_vp)]),
            ("colibri_tier_destroy", None, [_vp]),
            ("colibri_tier_stats", ctypes.c_int, [_vp, _vp, _vp]),
            ("colibri_tier_state", ctypes.c_int, [_vp, _vp, _vp, _vp]),
            ("colibri_tier_pin", ctypes.c_int, [_vp, _vp, _i32, _vp]),
            ("colibri_tier_workspace_bytes", ctypes.c_size_t, [_vp, _i32]),
            ("colibri_tier_forward", ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, ctypes.c_size_t,
                                                    _vp]),
            ("colibri_tier_verify_step", ctypes.c_int, [_vp, _i32, _vp, _i32, _vp, _i32, _vp,
                                                        ctypes.c_size_t, _vp, _vp, _vp])]:
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


_debug_lib = None
DBG_GATE, DBG_UP, DBG_DOWN = 0, 1, 2


@contextlib.contextmanager
def debug_partials(out: torch.Tensor, kind: int, o0: int, o1: int, r0: int, r1: int, nb: int):
    """Runs the calls in the block on the test-only library, which stores the
    int32 block partials of matrix `kind` (DBG_GATE / DBG_UP / DBG_DOWN),
    output rows [o0, o1), weight rows [r0, r1), blocks [0, nb) into out
    (int32, device; see include/colibri_debug.h)."""
    global _lib, _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
        _debug_lib.colibri_debug_partials.restype = ctypes.c_int
        _debug_lib.colibri_debug_partials.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _i32]
    assert out.dtype == torch.int32 and out.is_cuda and out.numel() >= (o1 - o0) * (r1 - r0) * nb
    _check(_debug_lib.colibri_debug_partials(_ptr(out), kind, o0, o1, r0, r1, nb), "colibri_debug_partials")
    saved, _lib = lib(), _debug_lib
    try:
        yield
    finally:
        _debug_lib.colibri_debug_partials(None, 0, 0, 0, 0, 0, 0)
        _lib = saved


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


def _bank_ptr(t: torch.Tensor):
    """Device memory, or pinned host memory (the slow tier of a tiered layer)."""
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError("device or pinned host tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------

@dataclass
class QBank:
    """n_mat quantised matrices [rows][K]: data uint8 [n_mat][rows][K*qtype/8],
    scales fp32 [n_mat][rows] or, with group > 0, [n_mat][rows * K/group]
    (device tensors)."""
    data: torch.Tensor
    scale: torch.Tensor
    qtype: int
    group: int = 0

    def desc(self) -> QBankDesc:
        n_mat, rows, rb = self.data.shape
        return QBankDesc(_bank_ptr(self.data), _bank_ptr(self.scale), n_mat, rows,
                         rb * 8 // self.qtype, self.qtype, self.group)


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


def moe_layer_forward_noalloc(layer: MoELayer, x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """out fp32 [S][hidden] = the layer applied to x, with the library's static
    per-GPU scratch as workspace (no allocation by the call; out is the
    caller's).  Batches whose workspace exceeds NOALLOC_SCRATCH_BYTES raise
    with COLI_E_SCRATCH."""
    _check(lib().colibri_moe_layer_forward_noalloc(ctypes.byref(layer.desc), _ptr(x), x.shape[0], _ptr(out),
                                                   _stream()), "colibri_moe_layer_forward_noalloc")
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


# ---------------------------------------------------------------------------
# Tiered expert residency: host-side slot cache and the tiered layer.

_u64 = ctypes.c_uint64
PLAN_SLOT_BITS = 11


class CacheLoad(ctypes.Structure):
    """coli_cache_load"""
    _fields_ = [("expert", _i32), ("slot", _i32), ("pass_", _i32), ("after", _i32)]


class CachePlan(ctypes.Structure):
    """coli_cache_plan"""
    _fields_ = [("n_pass", _i32), ("n_load", _i32), ("n_hit", _i32), ("n_miss", _i32)]


class CacheStats(ctypes.Structure):
    """coli_cache_stats"""
    _fields_ = [("plans", _u64), ("pairs", _u64), ("hits", _u64), ("misses", _u64),
                ("pin_loads", _u64), ("passes", _u64), ("prefetches", _u64), ("prefetch_loads", _u64),
                ("resident", _i32), ("pinned", _i32)]


def _i32_array(values):
    a = (_i32 * max(len(values), 1))()
    for i, v in enumerate(values):
        a[i] = int(v)
    return a


def _cache_stats(handle) -> dict:
    st = CacheStats()
    _check(lib().colibri_cache_stats(handle, ctypes.byref(st)), "colibri_cache_stats")
    return {f: getattr(st, f) for f, _ in CacheStats._fields_}


def _cache_state(handle, n_experts: int):
    slot_of = (_i32 * n_experts)()
    usage = (_u64 * n_experts)()
    _check(lib().colibri_cache_state(handle, slot_of, usage), "colibri_cache_state")
    return list(slot_of), list(usage)


class ExpertCache:
    """The host-side slot cache and planner (colibri_cache_*); needs no GPU."""

    def __init__(self, n_experts: int, n_slots: int):
        h = _vp()
        _check(lib().colibri_cache_create(n_experts, n_slots, ctypes.byref(h)), "colibri_cache_create")
        self._h, self.n_experts, self.n_slots = h, n_experts, n_slots

    def close(self):
        if self._h:
            lib().colibri_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def pin(self, experts: Sequence[int]):
        """-> [(expert, slot)] loads the pins need."""
        arr = _i32_array(experts)
        loads = (CacheLoad * max(len(experts), 1))()
        n = _i32(0)
        _check(lib().colibri_cache_pin(self._h, arr, len(experts), loads, ctypes.byref(n)),
               "colibri_cache_pin")
        return [(loads[i].expert, loads[i].slot) for i in range(n.value)]

    def unpin(self):
        lib().colibri_cache_unpin(self._h)

    def plan(self, ids: Sequence[int]) -> dict:
        """ids: routed expert ids (-1: dropped slot) -> codes, loads (expert,
        slot, pass, after), pass_pairs and the counts."""
        P = len(ids)
        m = min(P, self.n_experts)
        arr = _i32_array(ids)
        codes = (_i32 * max(P, 1))()
        loads = (CacheLoad * max(m, 1))()
        pp = (_i32 * (m + 1))()
        plan = CachePlan()
        _check(lib().colibri_cache_plan(self._h, arr, P, codes, loads, pp, ctypes.byref(plan)),
               "colibri_cache_plan")
        return {"codes": list(codes)[:P],
                "loads": [(loads[i].expert, loads[i].slot, loads[i].pass_, loads[i].after)
                          for i in range(plan.n_load)],
                "pass_pairs": list(pp)[:plan.n_pass], "n_pass": plan.n_pass, "n_hit": plan.n_hit,
                "n_miss": plan.n_miss}

    def prefetch(self, ids: Sequence[int]) -> dict:
        """Look-ahead prefetch of predicted ids -> loads (expert, slot, pass,
        after) and the counts."""
        P = len(ids)
        m = min(P, self.n_experts)
        arr = _i32_array(ids)
        loads = (CacheLoad * max(m, 1))()
        plan = CachePlan()
        _check(lib().colibri_cache_prefetch(self._h, arr, P, loads, ctypes.byref(plan)),
               "colibri_cache_prefetch")
        return {"loads": [(loads[i].expert, loads[i].slot, loads[i].pass_, loads[i].after)
                          for i in range(plan.n_load)],
                "n_pass": plan.n_pass, "n_hit": plan.n_hit, "n_miss": plan.n_miss}

    def stats(self) -> dict:
        return _cache_stats(self._h)

    def state(self):
        """-> (slot_of [E], usage [E])."""
        return _cache_state(self._h, self.n_experts)


class TieredLayer:
    """A layer whose routed experts live in pinned host memory (layer's
    gate/up/down QBanks on pinned CPU tensors) behind an HBM slot bank of
    n_slots experts (colibri_tier_*)."""

    def __init__(self, layer: MoELayer, n_slots: int):
        self.layer, self.n_slots = layer, n_slots
        nb = lib().colibri_tier_slot_bytes(ctypes.byref(layer.desc), n_slots)
        if nb == 0:
            raise ColibriError(COLI_E_INVAL, "colibri_tier_slot_bytes")
        self.slot_mem = torch.empty(nb, dtype=torch.uint8, device="cuda")
        h = _vp()
        _check(lib().colibri_tier_create(ctypes.byref(layer.desc), n_slots, _ptr(self.slot_mem), nb,
                                         ctypes.byref(h)), "colibri_tier_create")
        self._h = h

    def close(self):
        if self._h:
            lib().colibri_tier_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def pin(self, experts: Sequence[int]):
        arr = _i32_array(experts)
        _check(lib().colibri_tier_pin(self._h, arr, len(experts), _stream()), "colibri_tier_pin")

    def workspace_bytes(self, S: int) -> int:
        n = lib().colibri_tier_workspace_bytes(self._h, S)
        if n == 0:
            raise ColibriError(COLI_E_INVAL, "colibri_tier_workspace_bytes")
        return n

    def workspace(self, S: int) -> torch.Tensor:
        return torch.empty(self.workspace_bytes(S), dtype=torch.uint8, device="cuda")

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
        S = x.shape[0]
        out = torch.empty_like(x) if out is None else out
        ws = self.workspace(S) if ws is None else ws
        _check(lib().colibri_tier_forward(self._h, _ptr(x), S, _ptr(out), _ptr(ws), ws.numel(),
                                          _stream()), "colibri_tier_forward")
        return out

    def prefetch(self, x: torch.Tensor):
        """Look-ahead prefetch for activations x (S <= 8 tokens) predicting
        this layer's input; runs on the tier's copy stream."""
        _check(lib().colibri_tier_prefetch(self._h, _ptr(x), x.shape[0], _stream()), "colibri_tier_prefetch")

    def stats(self) -> dict:
        st = CacheStats()
        _check(lib().colibri_tier_stats(self._h, ctypes.byref(st), _stream()), "colibri_tier_stats")
        return {f: getattr(st, f) for f, _ in CacheStats._fields_}

    def state(self):
        """-> (slot_of [E], usage [E])."""
        E = self.layer.n_experts
        slot_of = (_i32 * E)()
        usage = (_u64 * E)()
        _check(lib().colibri_tier_state(self._h, slot_of, usage, _stream()), "colibri_tier_state")
        return list(slot_of), list(usage)


def tier_verify_step(tiers: Sequence[TieredLayer], x: torch.Tensor, out: torch.Tensor, ws: torch.Tensor,
                     union_mask: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None,
                     lookahead: bool = True):
    """One verify step through the tiers in order (colibri_tier_verify_step):
    x [n_layers][S][hidden] per-layer inputs, out [n_layers][S][hidden];
    union_mask int32 [n_layers][(E + 31) / 32] (zero before the first step)
    and stats int32 [n_layers][2] (distinct experts of the step, and how many
    of them the previous step used), both given or both None."""
    n = len(tiers)
    arr = (_vp * n)(*[t._h for t in tiers])
    _check(lib().colibri_tier_verify_step(arr, n, _ptr(x), x.shape[1], _ptr(out), 1 if lookahead else 0,
                                          _ptr(ws), ws.numel(), _ptr(union_mask), _ptr(stats), _stream()),
           "colibri_tier_verify_step")
    return out

"""ctypes binding of the oracle in coli_ref.c (argument marshalling only).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only importers.  The GPU package never
imports this module and this module never imports the GPU package.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "coli_ref.c")
LIB_PATH = os.path.join(HERE, "libcoli_ref.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-Wall", "-Wextra", "-fPIC", "-shared"]


def build() -> str:
    """Compile the oracle with gcc into oracle/libcoli_ref.so."""
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


class RefBank(ctypes.Structure):
    _fields_ = [("mat_data", ctypes.POINTER(ctypes.c_void_p)),
                ("mat_scale", ctypes.POINTER(ctypes.c_void_p)),
                ("n_mat", _i32), ("rows", _i32), ("K", _i32), ("bits", _i32), ("group", _i32)]


class RefRouteOpts(ctypes.Structure):
    _fields_ = [("n_group", _i32), ("topk_group", _i32), ("top_p", _f32)]


class RefLayer(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("inter", _i32), ("n_experts", _i32), ("top_k", _i32),
                ("routed_scaling_factor", _f32),
                ("router_w", _p), ("router_bias", _p),
                ("gate", RefBank), ("up", RefBank), ("down", RefBank),
                ("has_shared", _i32),
                ("sh_gate", RefBank), ("sh_up", RefBank), ("sh_down", RefBank),
                ("route", RefRouteOpts)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.ref_round_half_away.restype = _f32
        L.ref_round_half_away.argtypes = [_f32]
        L.ref_quantize_q8_0.argtypes = [_p, _i64, _p, _p]
        L.ref_row_bytes.restype = _i32
        L.ref_row_bytes.argtypes = [_i32, _i32]
        L.ref_weight_code.restype = _i32
        L.ref_weight_code.argtypes = [_p, _i32, _i32]
        L.ref_pack_row.argtypes = [_p, _i32, _i32, _p]
        L.ref_block_partial.restype = _i32
        L.ref_block_partial.argtypes = [_p, _i32, _p, _i32]
        L.ref_qdot.restype = _f32
        L.ref_qdot.argtypes = [_p, _i32, _f32, _p, _p, _i32]
        L.ref_qdot_f64.restype = ctypes.c_double
        L.ref_qdot_f64.argtypes = [_p, _i32, _f32, _p, _p, _i32]
        L.ref_qdot_grouped.restype = _f32
        L.ref_qdot_grouped.argtypes = [_p, _i32, _p, _i32, _p, _p, _i32]
        L.ref_qdot_grouped_f64.restype = ctypes.c_double
        L.ref_qdot_grouped_f64.argtypes = [_p, _i32, _p, _i32, _p, _p, _i32]
        L.ref_cexp.restype = _f32
        L.ref_cexp.argtypes = [_f32]
        L.ref_silu.restype = _f32
        L.ref_silu.argtypes = [_f32]
        L.ref_cexp_array.argtypes = [_p, _p, _i64]
        L.ref_silu_array.argtypes = [_p, _p, _i64]
        L.ref_expert_ffn.restype = ctypes.c_int
        L.ref_expert_ffn.argtypes = [ctypes.POINTER(RefBank)] * 3 + [_i32, _p, _p] + [_p] * 6
        L.ref_route_token.restype = ctypes.c_int
        L.ref_route_token.argtypes = [_p, _i32, _i32, _i32, _p, _p, _f32, _p, _p, _p, _p, _p]
        L.ref_route_token_opt.restype = ctypes.c_int
        L.ref_route_token_opt.argtypes = [_p, _i32, _i32, _i32, _p, _p, _f32, ctypes.POINTER(RefRouteOpts),
                                          _p, _p, _p, _p, _p]
        L.ref_dispatch.argtypes = [_p, _i32, _i32, _i32, _p, _p, _p, _p, _p]
        L.ref_moe_layer_forward.restype = ctypes.c_int
        L.ref_moe_layer_forward.argtypes = [ctypes.POINTER(RefLayer), _p, _i32, _p,
                                            _p, _p, _p, _p, _p, _p]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


# ---------------------------------------------------------------------------

def round_half_away(v: float) -> float:
    return lib().ref_round_half_away(v)


def quantize_q8_0(v):
    """v [..., K] fp32 -> (codes int8 [..., K], scales fp32 [..., K/32])."""
    v = _c(v, np.float32)
    assert v.shape[-1] % 32 == 0
    q = np.empty(v.shape, dtype=np.int8)
    d = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), dtype=np.float32)
    lib().ref_quantize_q8_0(_ptr(v), v.size, _ptr(q), _ptr(d))
    return q, d


def row_bytes(K: int, bits: int) -> int:
    return lib().ref_row_bytes(K, bits)


def weight_code(row, bits: int, col: int) -> int:
    row = _c(row, np.uint8)
    return lib().ref_weight_code(_ptr(row), bits, col)


def unpack_row(row, bits: int, K: int) -> np.ndarray:
    row = _c(row, np.uint8)
    return np.array([lib().ref_weight_code(_ptr(row), bits, c) for c in range(K)], dtype=np.int8)


def pack_row(codes, bits: int) -> np.ndarray:
    codes = _c(codes, np.int8)
    out = np.empty(row_bytes(codes.size, bits), dtype=np.uint8)
    lib().ref_pack_row(_ptr(codes), codes.size, bits, _ptr(out))
    return out


def block_partial(row, bits: int, q, b: int) -> int:
    row, q = _c(row, np.uint8), _c(q, np.int8)
    return lib().ref_block_partial(_ptr(row), bits, _ptr(q), b)


def qdot(row, bits: int, scale: float, q, d) -> float:
    row, q, d = _c(row, np.uint8), _c(q, np.int8), _c(d, np.float32)
    return lib().ref_qdot(_ptr(row), bits, scale, _ptr(q), _ptr(d), q.size)


def qdot_f64(row, bits: int, scale: float, q, d) -> float:
    row, q, d = _c(row, np.uint8), _c(q, np.int8), _c(d, np.float32)
    return lib().ref_qdot_f64(_ptr(row), bits, scale, _ptr(q), _ptr(d), q.size)


def qdot_grouped(row, bits: int, scales, group: int, q, d) -> float:
    """Row dot with one scale per `group` columns (scales [K/group])."""
    row, s, q, d = _c(row, np.uint8), _c(scales, np.float32), _c(q, np.int8), _c(d, np.float32)
    return lib().ref_qdot_grouped(_ptr(row), bits, _ptr(s), group, _ptr(q), _ptr(d), q.size)


def qdot_grouped_f64(row, bits: int, scales, group: int, q, d) -> float:
    row, s, q, d = _c(row, np.uint8), _c(scales, np.float32), _c(q, np.int8), _c(d, np.float32)
    return lib().ref_qdot_grouped_f64(_ptr(row), bits, _ptr(s), group, _ptr(q), _ptr(d), q.size)


def cexp(z) -> np.ndarray:
    z = _c(z, np.float32)
    out = np.empty_like(z)
    lib().ref_cexp_array(_ptr(z), _ptr(out), z.size)
    return out


def silu(g) -> np.ndarray:
    g = _c(g, np.float32)
    out = np.empty_like(g)
    lib().ref_silu_array(_ptr(g), _ptr(out), g.size)
    return out


# ---------------------------------------------------------------------------
# Banks and layers: accept the generator's Bank / Layer objects (CPU tensors)
# or plain lists of numpy arrays.

def _as_np(t):
    if t is None:
        return None
    if hasattr(t, "numpy"):
        t = t.detach().cpu().contiguous().numpy()
    return np.ascontiguousarray(t)


class _BankHandle:
    """Keeps the numpy arrays alive while the C structure points at them."""

    def __init__(self, n_mat, rows, K, bits, data, scale, group=0):
        self.data = [None if d is None else _c(_as_np(d), np.uint8) for d in data]
        self.scale = [None if s is None else _c(_as_np(s), np.float32) for s in scale]
        self.dp = (ctypes.c_void_p * n_mat)(*[None if d is None else d.ctypes.data for d in self.data])
        self.sp = (ctypes.c_void_p * n_mat)(*[None if s is None else s.ctypes.data for s in self.scale])
        self.c = RefBank(ctypes.cast(self.dp, ctypes.POINTER(ctypes.c_void_p)),
                         ctypes.cast(self.sp, ctypes.POINTER(ctypes.c_void_p)),
                         n_mat, rows, K, bits, group)


def bank(b) -> _BankHandle:
    """From a synth.Bank (or any object with n_mat/rows/K/bits/data/scale and,
    for group-wise scales, group)."""
    return _BankHandle(b.n_mat, b.rows, b.K, b.bits, b.data, b.scale, getattr(b, "group", 0))


def expert_ffn(gate, up, down, e: int, xq, xd):
    """One expert on one token.  Returns dict g, u, h, hq, hd, y."""
    G, U, D = (x if isinstance(x, _BankHandle) else bank(x) for x in (gate, up, down))
    I, H = G.c.rows, G.c.K
    xq, xd = _c(xq, np.int8), _c(xd, np.float32)
    out = dict(g=np.empty(I, np.float32), u=np.empty(I, np.float32), h=np.empty(I, np.float32),
               hq=np.empty(I, np.int8), hd=np.empty(I // 32, np.float32), y=np.empty(H, np.float32))
    st = lib().ref_expert_ffn(ctypes.byref(G.c), ctypes.byref(U.c), ctypes.byref(D.c), e,
                              _ptr(xq), _ptr(xd), _ptr(out["g"]), _ptr(out["u"]), _ptr(out["h"]),
                              _ptr(out["hq"]), _ptr(out["hd"]), _ptr(out["y"]))
    if st != 0:
        raise RuntimeError(f"ref_expert_ffn status {st}")
    return out


def route_opts(n_group: int = 1, topk_group: int = 1, top_p: float = 1.0) -> RefRouteOpts:
    return RefRouteOpts(n_group, topk_group, top_p)


def route_token(x, router_w, bias, k: int, rsf: float, opts: Optional[RefRouteOpts] = None):
    """One token.  Returns dict ids (-1: slot dropped by top-p), w (fp64), s, c,
    gap (smallest decision margin)."""
    x, W, b = _c(_as_np(x), np.float32), _c(_as_np(router_w), np.float32), _c(_as_np(bias), np.float32)
    E, H = W.shape
    ids = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    s = np.empty(E, np.float32)
    c = np.empty(E, np.float32)
    gap = np.empty(1, np.float32)
    if opts is None:
        st = lib().ref_route_token(_ptr(x), H, E, k, _ptr(W), _ptr(b), rsf,
                                   _ptr(ids), _ptr(w), _ptr(s), _ptr(c), _ptr(gap))
    else:
        st = lib().ref_route_token_opt(_ptr(x), H, E, k, _ptr(W), _ptr(b), rsf, ctypes.byref(opts),
                                       _ptr(ids), _ptr(w), _ptr(s), _ptr(c), _ptr(gap))
    if st != 0:
        raise RuntimeError(f"ref_route_token status {st}")
    return dict(ids=ids, w=w, s=s, c=c, gap=float(gap[0]))


def route(x, router_w, bias, k: int, rsf: float, opts: Optional[RefRouteOpts] = None):
    """All tokens of x [S][H]: ids [S][k], w [S][k] fp64, gaps [S]."""
    x = _c(_as_np(x), np.float32)
    res = [route_token(x[t], router_w, bias, k, rsf, opts) for t in range(x.shape[0])]
    S = x.shape[0]
    ids = np.array([r["ids"] for r in res], np.int32).reshape(S, k)
    w = np.array([r["w"] for r in res], np.float64).reshape(S, k)
    gaps = np.array([r["gap"] for r in res], np.float32)
    return ids, w, gaps


def dispatch(ids, E: int):
    """ids [S][k] -> dict offsets [E+1], sorted [S*k], inv [S*k], active, n_active."""
    ids = _c(ids, np.int32)
    S, k = ids.shape
    P = S * k
    offsets = np.empty(E + 1, np.int32)
    srt = np.empty(max(P, 1), np.int32)
    inv = np.empty(max(P, 1), np.int32)
    active = np.empty(E, np.int32)
    na = np.empty(1, np.int32)
    lib().ref_dispatch(_ptr(ids), S, k, E, _ptr(offsets), _ptr(srt), _ptr(inv),
                       _ptr(active), _ptr(na))
    n = int(na[0])
    return dict(offsets=offsets, sorted=srt[:P], inv=inv[:P], active=active[:n], n_active=n)


class LayerHandle:
    def __init__(self, layer):
        w = layer.w
        self.router_w = _c(_as_np(layer.router_w), np.float32)
        self.bias = _c(_as_np(layer.bias), np.float32)
        self.banks = [bank(layer.gate), bank(layer.up), bank(layer.down)]
        if w.has_shared:
            self.sh = [bank(layer.sh_gate), bank(layer.sh_up), bank(layer.sh_down)]
        else:
            self.sh = [self.banks[0]] * 3  # unused when has_shared == 0
        self.hidden, self.inter, self.k = w.hidden, w.inter, w.top_k
        self.c = RefLayer(w.hidden, w.inter, w.n_experts, w.top_k, w.rsf,
                          self.router_w.ctypes.data, self.bias.ctypes.data,
                          self.banks[0].c, self.banks[1].c, self.banks[2].c,
                          1 if w.has_shared else 0,
                          self.sh[0].c, self.sh[1].c, self.sh[2].c,
                          route_opts(w.n_group, w.topk_group, w.top_p))


def layer_forward(layer, x):
    """Whole layer on x [S][H].  Returns dict out (fp64), xq, xd, ids, w, y_routed, y_shared."""
    Lh = layer if isinstance(layer, LayerHandle) else LayerHandle(layer)
    x = _c(_as_np(x), np.float32)
    S, H = x.shape
    k = Lh.k
    r = dict(out=np.empty((S, H), np.float64), xq=np.empty((S, H), np.int8),
             xd=np.empty((S, H // 32), np.float32), ids=np.empty((S, k), np.int32),
             w=np.empty((S, k), np.float64), y_routed=np.empty((S * k, H), np.float32),
             y_shared=np.zeros((S, H), np.float32))
    st = lib().ref_moe_layer_forward(ctypes.byref(Lh.c), _ptr(x), S, _ptr(r["out"]),
                                     _ptr(r["xq"]), _ptr(r["xd"]), _ptr(r["ids"]), _ptr(r["w"]),
                                     _ptr(r["y_routed"]), _ptr(r["y_shared"]))
    if st != 0:
        raise RuntimeError(f"ref_moe_layer_forward status {st}")
    return r

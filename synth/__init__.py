"""Seeded synthetic inputs for the MoE-layer tests and benchmark.

This module holds none of the layer's arithmetic.  It has a counter-based
random generator and the recipes of the five workloads; both the GPU path and
the oracle receive exactly the tensors it produces.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: value i of a stream with
key K is mix64(K + (i + 1) * 0x9E3779B97F4A7C15), where mix64 is the
generator's output finaliser.  It is written with torch int64 operations
(wrapping multiply, masked logical shifts), so the same code gives the same
bits on the CPU and on a GPU.  Stream keys are FNV-1a-64 hashes of text labels,
so every tensor (and every expert's matrix) has its own stream and can be
generated on its own.

Real-valued draws (activations, router weights, row scales, biases) are made
on the CPU in float64 by Box-Muller and rounded to float32.  Packed weights
are raw random bytes: every byte is a valid pair of int4 nibbles (uniform on
[-8, 7]) or a valid quad of int2 values (uniform on [-2, 1]); int8 codes take
16 random bits each, mapped to [-127, 127] by multiply-shift.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _signed(v: int) -> int:
    v &= (1 << 64) - 1
    return v - (1 << 64) if v >= (1 << 63) else v


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    if s == 0:
        return z
    return (z >> s) & ((1 << (64 - s)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output finaliser on int64 bit patterns."""
    z = (z ^ _lsr(z, 30)) * _signed(_M1)
    z = (z ^ _lsr(z, 27)) * _signed(_M2)
    return z ^ _lsr(z, 31)


def mix64_int(x: int) -> int:
    """Pure-Python SplitMix64 finaliser (used to cross-check the tensor code)."""
    m = (1 << 64) - 1
    z = x & m
    z = ((z ^ (z >> 30)) * _M1) & m
    z = ((z ^ (z >> 27)) * _M2) & m
    return z ^ (z >> 31)


def stream_key(*labels) -> int:
    """64-bit stream key from text labels (FNV-1a-64 of the joined labels)."""
    text = "/".join(str(x) for x in labels).encode()
    h = 0xCBF29CE484222325
    for byte in text:
        h ^= byte
        h = (h * 0x100000001B3) & ((1 << 64) - 1)
    return mix64_int(h)


def random_u64(key: int, n: int, start: int = 0, device="cpu") -> torch.Tensor:
    """Values start .. start+n-1 of stream `key`, as int64 bit patterns."""
    idx = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return mix64(idx * _signed(_GOLDEN) + _signed(key))


_CHUNK = 1 << 24  # int64 words per generation chunk (128 MiB)


def random_bytes(key: int, nbytes: int, device="cpu") -> torch.Tensor:
    """nbytes random bytes of stream `key` (uint8 tensor), little-endian words."""
    nwords = (nbytes + 7) // 8
    out = torch.empty(nwords * 8, dtype=torch.uint8, device=device)
    words = out.view(torch.int64)
    for s in range(0, nwords, _CHUNK):
        n = min(_CHUNK, nwords - s)
        words[s:s + n] = random_u64(key, n, start=s, device=device)
    return out[:nbytes]


def random_int8_codes(key: int, n: int, device="cpu") -> torch.Tensor:
    """n int8 codes uniform on [-127, 127]: 16 random bits each, multiply-shift."""
    nwords = (n + 3) // 4
    out = torch.empty(nwords * 4, dtype=torch.int8, device=device)
    for s in range(0, nwords, _CHUNK):
        m = min(_CHUNK, nwords - s)
        w = random_u64(key, m, start=s, device=device)
        parts = []
        for lane in range(4):
            bits16 = _lsr(w, 16 * lane) & 0xFFFF
            parts.append(((bits16 * 255) >> 16) - 127)
        codes = torch.stack(parts, dim=1).reshape(-1).to(torch.int8)
        out[4 * s:4 * (s + m)] = codes
    return out[:n]


def uniform01(key: int, n: int) -> np.ndarray:
    """n float64 uniforms in (0, 1) from stream `key` (53 bits each, centred)."""
    w = random_u64(key, n).numpy().view(np.uint64)
    return ((w >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(key: int, n: int, std: float = 1.0) -> np.ndarray:
    """n float32 draws of N(0, std^2) by Box-Muller on stream `key`."""
    m = (n + 1) // 2
    u = uniform01(key, 2 * m)
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    t = 2.0 * math.pi * u[1::2]
    z = np.empty(2 * m, dtype=np.float64)
    z[0::2] = r * np.cos(t)
    z[1::2] = r * np.sin(t)
    return (z[:n] * std).astype(np.float32)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic MoE layer plus a batch size.

    `var_*` fields are variances: N(0, a) is read as mean 0, variance a.
    """
    name: str
    layer: str          # weight-stream label: workloads naming the same layer share weights
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    rsf: float
    has_shared: bool
    bits: int
    S: int
    var_router: float
    bias_kind: str      # "normal" or "zipf"
    var_bias: float = 0.0
    zipf_s: float = 1.1
    zipf_beta: float = 0.1
    scale_mult: float = 0.02
    seed: int = 0
    # router variants (1, 1, 1.0: plain top-k)
    n_group: int = 1
    topk_group: int = 1
    top_p: float = 1.0
    # columns per weight scale in every bank (0: one scale per row)
    group: int = 0

    def row_bytes(self, K: int) -> int:
        return K * self.bits // 8


def _glm(name, layer, bits, S, bias_kind="normal", var_bias=1e-4):
    return Workload(name=name, layer=layer, hidden=6144, inter=2048, n_experts=256,
                    top_k=8, rsf=2.5, has_shared=True, bits=bits, S=S,
                    var_router=1.0 / 6144, bias_kind=bias_kind, var_bias=var_bias)


WORKLOADS: Dict[str, Workload] = {
    # Tiny layer: H=256, 16 experts of I=128, top-2, rsf 1.0, no shared, int8, S=8.
    "tiny": Workload(name="tiny", layer="tiny_int8", hidden=256, inter=128, n_experts=16,
                     top_k=2, rsf=1.0, has_shared=False, bits=8, S=8,
                     var_router=1.0 / 256, bias_kind="normal", var_bias=0.1),
    # GLM-5.2-shaped layer (H=6144, 256 experts of I=2048, top-8, rsf 2.5, shared).
    "decode": _glm("decode", "glm_int4", 4, 1),
    "prefill": _glm("prefill", "glm_int4", 4, 512),
    "verify": _glm("verify", "glm_int8", 8, 4),
    "skewed": _glm("skewed", "glm_int2", 2, 2048, bias_kind="zipf"),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (for small parity cases)."""
    return dataclasses.replace(w, **changes)


@dataclasses.dataclass
class Bank:
    """n_mat matrices [rows][K] packed at `bits`, with per-row fp32 scales.

    data[m] / scale[m] are tensors for matrix m, or None when not generated.
    """
    n_mat: int
    rows: int
    K: int
    bits: int
    data: List[Optional[torch.Tensor]]
    scale: List[Optional[torch.Tensor]]
    # When every matrix is generated: one contiguous [n_mat][rows][row_bytes]
    # uint8 tensor and one [n_mat][rows] fp32 tensor that data/scale view.
    storage: Optional[torch.Tensor] = None
    scale_storage: Optional[torch.Tensor] = None
    # columns per scale (0: scale[m] holds one value per row; else rows * K/group
    # values, row r's at r * K/group)
    group: int = 0


@dataclasses.dataclass
class Layer:
    w: Workload
    router_w: torch.Tensor   # [E][H] fp32
    bias: torch.Tensor       # [E] fp32
    gate: Bank
    up: Bank
    down: Bank
    sh_gate: Optional[Bank]
    sh_up: Optional[Bank]
    sh_down: Optional[Bank]


def _key(w: Workload, *labels) -> int:
    return stream_key("colibri-synth", w.seed, *labels)


def router_weights(w: Workload) -> torch.Tensor:
    E, H = w.n_experts, w.hidden
    z = normal(_key(w, w.layer, "router_w"), E * H, std=math.sqrt(w.var_router))
    return torch.from_numpy(z.reshape(E, H))


def router_bias(w: Workload) -> torch.Tensor:
    E = w.n_experts
    if w.bias_kind == "normal":
        return torch.from_numpy(normal(_key(w, w.layer, "bias"), E, std=math.sqrt(w.var_bias)))
    # Zipf popularity: a seeded permutation gives expert e the popularity rank
    # r(e) in 1..E; its bias is beta * ln(p_r / p_1) with p_r proportional to
    # r^-s, i.e. -beta * s * ln r(e).
    order = np.argsort(random_u64(_key(w, w.layer, "zipf_perm"), E).numpy().view(np.uint64),
                       kind="stable")
    rank = np.empty(E, dtype=np.int64)
    rank[order] = np.arange(1, E + 1)
    b = -w.zipf_beta * w.zipf_s * np.log(rank.astype(np.float64))
    return torch.from_numpy(b.astype(np.float32))


def _mat_bytes(w: Workload, name: str, m: int, rows: int, K: int, device) -> torch.Tensor:
    key = _key(w, w.layer, name, m)
    n = rows * K * w.bits // 8
    if w.bits == 8:
        return random_int8_codes(key, n, device=device).view(torch.uint8).view(rows, -1)
    return random_bytes(key, n, device=device).view(rows, -1)


def _mat_scale(w: Workload, name: str, m: int, rows: int) -> torch.Tensor:
    z = normal(_key(w, w.layer, name + "_scale", m), rows)
    return torch.from_numpy(np.abs(z) * np.float32(w.scale_mult))


def make_bank(w: Workload, name: str, n_mat: int, rows: int, K: int,
              experts=None, device="cpu") -> Bank:
    """Generate a bank; `experts` limits which matrices are materialised.
    Scales: rows values per matrix, or rows * K/group with group-wise scales
    (the same |N(0, 1)| * scale_mult recipe per value)."""
    data: List[Optional[torch.Tensor]] = [None] * n_mat
    scale: List[Optional[torch.Tensor]] = [None] * n_mat
    rb = K * w.bits // 8
    ns = rows * (K // w.group) if w.group else rows
    if experts is None:
        storage = torch.empty(n_mat, rows, rb, dtype=torch.uint8, device=device)
        scale_storage = torch.empty(n_mat, ns, dtype=torch.float32, device=device)
        for m in range(n_mat):
            storage[m] = _mat_bytes(w, name, m, rows, K, device)
            scale_storage[m] = _mat_scale(w, name, m, ns).to(device)
            data[m] = storage[m]
            scale[m] = scale_storage[m]
        return Bank(n_mat, rows, K, w.bits, data, scale, storage, scale_storage, w.group)
    for m in sorted(set(int(e) for e in experts)):
        data[m] = _mat_bytes(w, name, m, rows, K, device)
        scale[m] = _mat_scale(w, name, m, ns).to(device)
    return Bank(n_mat, rows, K, w.bits, data, scale, group=w.group)


def make_layer(w: Workload, experts=None, device="cpu") -> Layer:
    """The workload's layer.  `experts` (optional) limits the routed experts
    materialised (the oracle only needs the ones a computation touches)."""
    E, H, I = w.n_experts, w.hidden, w.inter
    gate = make_bank(w, "gate", E, I, H, experts, device)
    up = make_bank(w, "up", E, I, H, experts, device)
    down = make_bank(w, "down", E, H, I, experts, device)
    if w.has_shared:
        sg = make_bank(w, "sh_gate", 1, I, H, None, device)
        su = make_bank(w, "sh_up", 1, I, H, None, device)
        sd = make_bank(w, "sh_down", 1, H, I, None, device)
    else:
        sg = su = sd = None
    return Layer(w, router_weights(w).to(device), router_bias(w).to(device),
                 gate, up, down, sg, su, sd)


def token_activation(w: Workload, t: int, attempt: int = 0, tag: str = "") -> torch.Tensor:
    """Token t's fp32 activation row, draw number `attempt` (N(0, 1))."""
    return torch.from_numpy(normal(_key(w, "x", w.name + tag, t, attempt), w.hidden))


def activations(w: Workload, S: Optional[int] = None,
                attempts: Optional[Dict[int, int]] = None, tag: str = "") -> torch.Tensor:
    """[S][H] fp32 activations; attempts[t] selects a redraw of token t."""
    S = w.S if S is None else S
    attempts = attempts or {}
    if S == 0:
        return torch.zeros(0, w.hidden)
    return torch.stack([token_activation(w, t, attempts.get(t, 0), tag) for t in range(S)])

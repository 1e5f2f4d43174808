"""Builder for the hand-worked two-expert layer of tests/golden/hand_two_expert.json.

Constructs the inputs from the fixture's rules and evaluates its closed form
(exact rational arithmetic; no blocks, no fold order, no exp).
"""

import json
import os
from fractions import Fraction

import numpy as np
import torch

import synth

FIXTURE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_two_expert.json")
H = I = 64
E = 2


def load():
    with open(FIXTURE) as f:
        return json.load(f)


def x_values():
    x = np.array([i - 32 for i in range(H)], dtype=np.float32)
    x[0], x[32] = 127.0, -127.0
    return x


def _on(e, i):
    return i % 32 == 0 or (i + e) % 3 != 0


def _up_col(e, i):
    return 0 if i in (0, 32) else (7 * i + e) % 64


def _sigma(e, i):
    return 1 if (i + e) % 2 == 0 else -1


def gate_codes(e):
    c = np.zeros((I, H), np.int8)
    s = np.zeros(I, np.float32)
    for i in range(I):
        if _on(e, i):
            c[i, 0], s[i] = 1, 0.25
        else:
            c[i, 32], s[i] = 1, 1.0
    return c, s


def up_codes(e):
    c = np.zeros((I, H), np.int8)
    s = np.full(I, 0.125, np.float32)
    for i in range(I):
        c[i, _up_col(e, i)] = _sigma(e, i)
    return c, s


def down_codes(e):
    c = np.zeros((H, I), np.int8)
    s = np.zeros(H, np.float32)
    for n in range(H):
        c[n, n] += 1
        c[n, (n + 17 + e) % 64] -= 1
        s[n] = 2.0 ** -(n % 3)
    return c, s


def hq_closed(e):
    x = x_values()
    return [(_sigma(e, i) * int(x[_up_col(e, i)])) if _on(e, i) else 0 for i in range(I)]


def y_closed(e):
    hq = hq_closed(e)
    return [Fraction(1, 2 ** (n % 3)) * Fraction(127, 32) * (hq[n] - hq[(n + 17 + e) % 64])
            for n in range(H)]


def out_closed(with_shared=False):
    y0, y1 = y_closed(0), y_closed(1)
    out = [Fraction(5, 4) * (a + b) for a, b in zip(y0, y1)]
    if with_shared:
        out = [o + a for o, a in zip(out, y0)]
    return out


def _pack(codes, bits):
    import oracle
    return np.stack([oracle.pack_row(r, bits) for r in codes])


def layer(bits=8, bias=(0.0, 0.0), with_shared=False):
    """A synth.Layer holding the example, packed at `bits` (8, 4 or 2)."""
    w = synth.Workload(name="hand", layer="hand", hidden=H, inter=I, n_experts=E, top_k=2,
                       rsf=2.5, has_shared=with_shared, bits=bits, S=1, var_router=0.0,
                       bias_kind="normal")
    mats = {"gate": [], "up": [], "down": []}
    scales = {"gate": [], "up": [], "down": []}
    for e in range(E):
        for name, fn in (("gate", gate_codes), ("up", up_codes), ("down", down_codes)):
            c, s = fn(e)
            mats[name].append(torch.from_numpy(_pack(c, bits)))
            scales[name].append(torch.from_numpy(s))

    def bank(name, idx):
        data = [mats[name][i] for i in idx]
        sc = [scales[name][i] for i in idx]
        rows, K = (I, H) if name != "down" else (H, I)
        st = torch.stack(data).contiguous()
        ss = torch.stack(sc).contiguous()
        return synth.Bank(len(idx), rows, K, bits, [st[i] for i in range(len(idx))],
                          [ss[i] for i in range(len(idx))], st, ss)

    router_w = torch.full((E, H), 1.0 / 64, dtype=torch.float32)
    b = torch.tensor(bias, dtype=torch.float32)
    sh = [bank(n, [0]) for n in ("gate", "up", "down")] if with_shared else [None] * 3
    return synth.Layer(w, router_w, b, bank("gate", [0, 1]), bank("up", [0, 1]),
                       bank("down", [0, 1]), *sh)

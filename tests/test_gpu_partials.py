"""The int32 block partials themselves, dumped by the test-only build of the
same kernels (include/colibri_debug.h), against the oracle's
ref_block_partial bit for bit ("Show HN: 如何在我的低配置电脑上运行 GLM-5.2",
section 已实现的功能, integer dot-product item: exact integer block sums).

Every kernel family is covered: the one-token gate/up jobs (routed and the
shared expert's one-wave jobs), the fused one-token down + combine, the
separate one-token down kernel, the whole-row kernels for units of up to four
tokens, and both matrix-core K loops (the aligned one and the general one).
Weights take the extremes of each container's range and activation blocks
have codes of +-127."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import GAP, say, to_device

pytestmark = pytest.mark.gpu

SENTINEL = -(2 ** 31)
RANGES = {8: (-127, 127), 4: (-8, 7), 2: (-2, 1)}


@pytest.fixture(scope="module")
def qre():
    import quantized_routed_expert_sigmoid_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.lib()
    return m


def _extreme_bank(b: synth.Bank, seed: int):
    """Fills the bank with codes drawn from {lo, hi} of its width (and, for one
    row in eight, a row of lo only), packed by the oracle."""
    lo, hi = RANGES[b.bits]
    rng = np.random.default_rng(seed)
    for m in range(b.n_mat):
        codes = rng.choice(np.array([lo, hi], np.int8), size=(b.rows, b.K))
        codes[::8] = lo
        packed = np.stack([oracle.pack_row(codes[r], b.bits) for r in range(b.rows)])
        b.storage[m].copy_(torch.from_numpy(packed))


def _extreme_activations(w, S, tag):
    """Activations whose even 32-blocks are +-1 (codes +-127) and odd blocks
    normal draws, redrawn until the oracle's routing gaps exceed GAP."""
    L_router = synth.router_weights(w).numpy()
    bias = synth.router_bias(w).numpy()
    for attempt in range(50):
        x = synth.activations(w, S, tag=f"{tag}{attempt}").numpy().copy()
        xb = x.reshape(S, -1, 32)
        xb[:, ::2, :] = np.where(xb[:, ::2, :] >= 0, 1.0, -1.0)
        x = xb.reshape(S, -1)
        opts = oracle.route_opts(w.n_group, w.topk_group, w.top_p)
        if all(oracle.route_token(x[t], L_router, bias, w.top_k, w.rsf, opts)["gap"] > GAP for t in range(S)):
            return x
    raise AssertionError("no gapped activations")


def _rows_of(w, L, x, one_token):
    """Per output row o: (token, expert bank index or 'sh')."""
    S, k = x.shape[0], w.top_k
    ids, _, _ = oracle.route(x, L.router_w, L.bias, k, w.rsf, oracle.route_opts(w.n_group, w.topk_group, w.top_p))
    if one_token:
        rows = [(0, int(ids[0, u])) for u in range(k)]
        return rows + ([(0, "sh")] if w.has_shared else [])
    d = oracle.dispatch(ids, w.n_experts)
    rows = [(int(p) // k, int(ids[int(p) // k, int(p) % k])) for p in d["sorted"]]
    return rows + ([(t, "sh") for t in range(S)] if w.has_shared else [])


def _check_slice(qre, dev, w, L, x, kind, r0, r1, one_token, what):
    S = x.shape[0]
    rows = _rows_of(w, L, x, one_token)
    o0, o1 = 0, len(rows)
    K = w.hidden if kind != qre.DBG_DOWN else w.inter
    nb = K // 32
    out = torch.full(((o1 - o0) * (r1 - r0) * nb,), SENTINEL, dtype=torch.int32, device="cuda")
    xd = torch.from_numpy(x).cuda().contiguous()
    with qre.debug_partials(out, kind, o0, o1, r0, r1, nb):
        qre.moe_layer_forward(dev, xd)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(o1 - o0, r1 - r0, nb)
    xq, xdd = zip(*[oracle.quantize_q8_0(x[t]) for t in range(S)])
    n_cmp = 0
    for o, (t, e) in enumerate(rows):
        sh = e == "sh"
        gate, up, down = (L.sh_gate, L.sh_up, L.sh_down) if sh else (L.gate, L.up, L.down)
        m = 0 if sh else e
        if kind == qre.DBG_DOWN:
            q = oracle.expert_ffn(gate, up, down, m, xq[t], xdd[t])["hq"]
            bank = down
        else:
            q = xq[t]
            bank = gate if kind == qre.DBG_GATE else up
        for r in range(r0, r1):
            row = bank.data[m][r].numpy()
            want = [oracle.block_partial(row, bank.bits, q, b) for b in range(nb)]
            assert got[o, r - r0].tolist() == want, f"{what}: output row {o} (token {t}, expert {e}) weight row {r}"
            n_cmp += nb
    return n_cmp


# name: (workload changes, batch, kinds with their weight-row windows, one-token)
CASES = {
    # one token, shared expert as one-wave jobs, fused down + combine
    "decode": (dict(hidden=512, inter=256, n_experts=16, top_k=4, has_shared=True, var_router=1.0 / 512), 1,
               True),
    # one token, 33 units: the separate one-token down kernel
    "decode_many_units": (dict(hidden=256, inter=128, n_experts=40, top_k=32, has_shared=True,
                               var_router=1.0 / 256), 1, True),
    # units of up to four tokens on the whole-row kernels
    "small_batch": (dict(hidden=512, inter=256, n_experts=8, top_k=2, has_shared=True, var_router=1.0 / 512), 5,
                    False),
    # experts with >= 8 tokens on the matrix cores: aligned loop for gate/up
    # (H = 512), general loop for down (I = 256 at int4/int2; int8 aligned)
    "mfma": (dict(hidden=512, inter=256, n_experts=2, top_k=1, has_shared=True, var_router=1.0 / 512), 40, False),
    # the general loop with a ragged row (H = 288: nine blocks)
    "mfma_ragged": (dict(hidden=288, inter=96, n_experts=2, top_k=2, has_shared=False, var_router=1.0 / 288), 24,
                    False),
    # rows of 100 blocks (four chunks, the last ragged): int8 rows of four
    # chunks or more are loaded in half blocks by every GEMV kernel
    "decode_long_rows": (dict(hidden=3200, inter=3200, n_experts=4, top_k=4, has_shared=True,
                              var_router=1.0 / 3200), 1, True),
    "small_batch_long_rows": (dict(hidden=3200, inter=3200, n_experts=4, top_k=2, has_shared=True,
                                   var_router=1.0 / 3200), 5, False),
}
WINDOWS = {"gate": (0, 32), "up": (16, 48), "down": (56, 104)}


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("case", sorted(CASES))
def test_block_partials_bit_exact(qre, case, bits):
    kw, S, one_token = CASES[case]
    w = synth.scaled(synth.WORKLOADS["tiny"], name=f"pt_{case}_{bits}", layer=f"pt_{case}_{bits}", bits=bits, S=S,
                     **kw)
    L = synth.make_layer(w)
    for i, b in enumerate([L.gate, L.up, L.down] + ([L.sh_gate, L.sh_up, L.sh_down] if w.has_shared else [])):
        _extreme_bank(b, seed=1000 * bits + i)
    dev = to_device(L)
    x = _extreme_activations(w, S, tag=f"pt{case}")
    n = 0
    for name, kind in (("gate", qre.DBG_GATE), ("up", qre.DBG_UP), ("down", qre.DBG_DOWN)):
        rows = w.inter if kind != qre.DBG_DOWN else w.hidden
        r0, r1 = WINDOWS[name]
        r0, r1 = min(r0, rows), min(r1, rows)
        say(f"partials {case} int{bits} {name} rows [{r0}, {r1})")
        n += _check_slice(qre, dev, w, L, x, kind, r0, r1, one_token, f"{case} int{bits} {name}")
    assert n > 0

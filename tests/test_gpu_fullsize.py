"""GPU parity at the workloads' full sizes.

Layer level, in the launch configuration the benchmark times (one
colibri_moe_layer_forward over the whole batch): routing ids for every
token, and complete output rows for every token at S <= 4 and, at S = 512
and S = 2048, for a sample that holds random tokens, the last token of each
of the 8 most loaded experts (their ragged last matrix-core unit) and tokens
of experts with fewer than 8 tokens (at these sizes, with 8 or more pairs per
expert on average, the layer runs them on the matrix cores too).

Unit level, at S = 512 and S = 2048, through the stage calls over the whole
batch (route, dispatch, expert FFN): the expert outputs y, which are
bit-exact, of one token from every matrix-core unit and the last token of
the 8 most loaded experts (S = 2048: about 200 units) or of every expert
on the matrix cores (S = 512, where each holds one or two units), every
token of up to 12 experts on GEMV units, and one token from every unit of
the shared expert.  The oracle runs
only on the experts these rows need (copied from the device-generated layer:
the generator gives the same bits on both)."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import assert_close_rms, gapped_activations, say, to_device

pytestmark = pytest.mark.gpu

_LAYERS = {}
_X = {}
MFMA_MIN, MFMA_UNIT = 8, 32  # stage calls: experts with >= 8 tokens run in units of 32 on the matrix cores
N_THREADS = 16               # oracle calls release the GIL


@pytest.fixture(scope="module")
def qre():
    import quantized_routed_expert_sigmoid_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.lib()
    return m


def _device_layer(w):
    """Full layer generated on the GPU (cached per weight stream)."""
    if w.layer not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        say(f"generating layer {w.layer} on the GPU")
        _LAYERS[w.layer] = synth.make_layer(w, device="cuda")
        torch.cuda.synchronize()
    return _LAYERS[w.layer]


def _activations(w, Lg):
    if w.name not in _X:
        x, attempts = gapped_activations(w, Lg.router_w.cpu(), Lg.bias.cpu())
        say(f"  {w.name}: redrawn tokens {len(attempts)}")
        _X[w.name] = x
    return _X[w.name]


def _cpu_subset(Lg, experts):
    """The device layer with only `experts` (and the shared expert) copied to
    host memory, as the oracle takes it."""
    def sub(b):
        data = [b.storage[m].cpu() if m in experts else None for m in range(b.n_mat)]
        scale = [b.scale_storage[m].cpu() if m in experts else None for m in range(b.n_mat)]
        return synth.Bank(b.n_mat, b.rows, b.K, b.bits, data, scale, group=b.group)

    def full(b):
        return None if b is None else synth.Bank(b.n_mat, b.rows, b.K, b.bits, [b.storage[0].cpu()],
                                                 [b.scale_storage[0].cpu()], group=b.group)
    return synth.Layer(Lg.w, Lg.router_w.cpu(), Lg.bias.cpu(), sub(Lg.gate), sub(Lg.up), sub(Lg.down),
                       full(Lg.sh_gate), full(Lg.sh_up), full(Lg.sh_down))


def _expert_positions(ids_ref, E):
    """Sorted positions of each expert (pairs in ascending pair index)."""
    d = oracle.dispatch(ids_ref, E)
    off = d["offsets"]
    return d, {e: list(range(int(off[e]), int(off[e + 1]))) for e in range(E) if off[e + 1] > off[e]}


def _hot_experts(pos, n=8):
    return sorted(pos, key=lambda e: (-len(pos[e]), e))[:n]


@pytest.mark.parametrize("name,n_sample", [("decode", None), ("verify", None), ("prefill", 6), ("skewed", 6)])
def test_full_size_layer(qre, name, n_sample):
    w = synth.WORKLOADS[name]
    say(f"full-size {name}: S={w.S} bits={w.bits}")
    Lg = _device_layer(w)
    x = _activations(w, Lg)
    dev = to_device(Lg)
    xg = x.cuda()
    ids, wts = qre.route(dev, xg)
    out = qre.moe_layer_forward(dev, xg)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isfinite(out).all()

    router_w, bias = Lg.router_w.cpu(), Lg.bias.cpu()
    ids_ref, w_ref, _ = oracle.route(x.numpy(), router_w, bias, w.top_k, w.rsf)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(wts.cpu().numpy(), w_ref, rtol=2e-6, atol=1e-7)

    if n_sample is None:
        tokens = list(range(w.S))
    else:
        rng = np.random.default_rng(0)
        tokens = set(rng.choice(w.S, size=n_sample, replace=False).tolist())
        d, pos = _expert_positions(ids_ref, w.n_experts)
        srt = d["sorted"]
        # the last token of each of the 8 most loaded experts (ragged last unit)
        for e in _hot_experts(pos):
            tokens.add(int(srt[pos[e][-1]]) // w.top_k)
        # tokens of experts with fewer than 8 tokens (single small matrix-core units)
        small = [e for e in sorted(pos) if len(pos[e]) < MFMA_MIN][:3]
        for e in small:
            tokens.add(int(srt[pos[e][0]]) // w.top_k)
        tokens = sorted(tokens)
    needed = set(ids_ref[tokens].reshape(-1).tolist())
    say(f"  oracle on {len(tokens)} tokens ({len(needed)} experts)")
    Lc = _cpu_subset(Lg, needed)
    Lh = oracle.LayerHandle(Lc)
    xs = x.numpy()

    def one(t):
        return oracle.layer_forward(Lh, xs[t:t + 1])

    with ThreadPoolExecutor(N_THREADS) as ex:
        refs = list(ex.map(one, tokens))
    ref_out = np.concatenate([r["out"] for r in refs])
    assert np.array_equal(np.concatenate([r["ids"] for r in refs]), ids_ref[tokens])
    rel = assert_close_rms(out[tokens], ref_out, name)
    say(f"  max|diff|/rms = {rel:.3e}")


@pytest.mark.parametrize("name,n_hot", [("prefill", None), ("skewed", 8)])
def test_full_size_units(qre, name, n_hot):
    w = synth.WORKLOADS[name]
    S, k, E = w.S, w.top_k, w.n_experts
    say(f"full-size units {name}: S={S} bits={w.bits}")
    Lg = _device_layer(w)
    x = _activations(w, Lg)
    dev = to_device(Lg)
    xg = x.cuda()
    ids, _ = qre.route(dev, xg)
    offsets, srt_g, _, _ = qre.moe_dispatch(ids, E)
    xq, xd = qre.quantize_q8_0(xg)
    y = qre.expert_ffn_q(dev.gate, dev.up, dev.down, xq, xd, offsets, srt_g, k)
    sh_off = torch.tensor([0, S], dtype=torch.int32, device="cuda")
    ident = torch.arange(S, dtype=torch.int32, device="cuda")
    y_sh = qre.expert_ffn_q(*dev.shared, xq, xd, sh_off, ident, 1)
    torch.cuda.synchronize()

    ids_ref, _, _ = oracle.route(x.numpy(), Lg.router_w.cpu(), Lg.bias.cpu(), k, w.rsf)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    d, pos = _expert_positions(ids_ref, E)
    srt = d["sorted"]
    assert np.array_equal(srt_g.cpu().numpy(), srt)

    # (sorted position, expert): one per matrix-core unit of the hot experts
    # and each one's last position; every position of GEMV-unit experts
    rows = []
    hot = _hot_experts(pos, n_hot) if n_hot else [e for e in sorted(pos) if len(pos[e]) >= MFMA_MIN]
    for e in hot:
        p = pos[e]
        assert len(p) >= MFMA_MIN, (e, len(p))
        rows += [(p[u], e) for u in range(0, len(p), MFMA_UNIT)] + [(p[-1], e)]
    small = [e for e in sorted(pos) if len(pos[e]) < MFMA_MIN]
    for e in small[:12]:
        rows += [(q, e) for q in pos[e]]
    rows = sorted(set(rows))
    sh_tokens = sorted(set(list(range(0, S, MFMA_UNIT)) + [S - 1]))
    n_units = sum((len(pos[e]) + MFMA_UNIT - 1) // MFMA_UNIT for e in hot)
    say(f"  {len(rows)} routed rows ({n_units} matrix-core units of {len(hot)} experts, "
        f"{min(len(small), 12)} GEMV-unit experts), {len(sh_tokens)} shared rows")

    needed = set(e for _, e in rows)
    Lc = _cpu_subset(Lg, needed)
    G, U, D = oracle.bank(Lc.gate), oracle.bank(Lc.up), oracle.bank(Lc.down)
    SG, SU, SD = oracle.bank(Lc.sh_gate), oracle.bank(Lc.sh_up), oracle.bank(Lc.sh_down)
    xs = x.numpy()
    q8 = {}

    def codes(t):
        if t not in q8:
            q8[t] = oracle.quantize_q8_0(xs[t])
        return q8[t]

    for t in set(int(srt[p]) // k for p, _ in rows) | set(sh_tokens):
        codes(t)

    def routed(item):
        p, e = item
        t = int(srt[p]) // k
        return oracle.expert_ffn(G, U, D, e, *codes(t))["y"]

    def shared(t):
        return oracle.expert_ffn(SG, SU, SD, 0, *codes(t))["y"]

    with ThreadPoolExecutor(N_THREADS) as ex:
        y_ref = list(ex.map(routed, rows))
        ysh_ref = list(ex.map(shared, sh_tokens))
    y = y.cpu().numpy()
    y_sh = y_sh.cpu().numpy()
    for (p, e), yr in zip(rows, y_ref):
        assert y[p].tobytes() == yr.tobytes(), f"{name}: sorted position {p} (expert {e}) differs"
    for t, yr in zip(sh_tokens, ysh_ref):
        assert y_sh[t].tobytes() == yr.tobytes(), f"{name}: shared expert, token {t} differs"

"""Tiered expert residency on the GPU (colibri_tier_* through the C ABI):
the routed experts live in pinned host memory behind a slot bank of a few
experts in HBM.  Every tiered forward must equal the resident forward on the
same weights bit for bit -- over sequences of batches that hit, miss, evict
and reload slots, with chunked passes when a batch needs more experts than
there are slots, with pinned experts, top-p-dropped slots and a shared
expert at another width -- and one case is checked against the oracle
directly.  After every forward the device planner's state (slot map, usage,
counters) must equal that of the host planner (colibri_cache_*, itself
checked on the CPU against the documented policy) fed the same routed ids."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import assert_close_rms, gapped_activations, say, to_device, to_slow_tier

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qre():
    import quantized_routed_expert_sigmoid_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.lib()
    return m


TIER_CASES = {
    # one token: the resident forward runs the fused decode kernels
    "decode_int4": dict(name="tdec4", layer="dec4", bits=4, hidden=512, inter=256, n_experts=64, top_k=6,
                        S=1, has_shared=True, rsf=2.5, var_router=1.0 / 512, var_bias=1e-4),
    "long_int4_shared": dict(name="tl4", layer="tiny_int4", bits=4, S=37, has_shared=True),
    "mfma_int4": dict(name="tmf4", layer="mf4", bits=4, hidden=512, inter=256, n_experts=8, top_k=2, S=64,
                      has_shared=True, rsf=2.5, var_router=1.0 / 512, var_bias=1e-4),
    "small_topp_groups": dict(name="trvs", layer="rvs", bits=8, n_experts=32, top_k=4, S=6,
                              has_shared=True, n_group=4, topk_group=2, top_p=0.8),
    "many_slots_int2": dict(name="tm2", layer="tm2", bits=2, hidden=256, inter=96, n_experts=64, top_k=16,
                            S=3, has_shared=False, var_router=1.0 / 256),
    # group-wise weight scales: the slot bank carries K/group scales per row
    "grouped_int4": dict(name="tg4", layer="gd4", bits=4, hidden=512, inter=256, n_experts=64, top_k=6,
                         S=1, has_shared=True, rsf=2.5, var_router=1.0 / 512, group=128),
}
SLOTS = {"decode_int4": [1, 8, 64], "long_int4_shared": [1, 3, 16], "mfma_int4": [1, 3, 8],
         "small_topp_groups": [2, 9], "many_slots_int2": [2, 17, 40], "grouped_int4": [2, 12]}
# batch order with repeats, so that later batches hit what earlier ones loaded
ORDER = [0, 1, 0, 2, 1, 0, 3]


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def _run_sequence(qre, w, dev, tier, order=ORDER, S=None, host=None):
    """Runs the batches through the tier and the resident layer; `host` (an
    ExpertCache mirroring the tier) is planned with the same routed ids."""
    S = w.S if S is None else S
    xs = {}
    misses = 0
    for b in order:
        if b not in xs:
            xs[b] = synth.activations(w, S, tag=f"tier{b}").cuda()
        before = tier.stats()["misses"]
        ref = qre.moe_layer_forward(dev, xs[b])
        got = tier.forward(xs[b])
        torch.cuda.synchronize()
        assert bits_equal(got, ref), f"batch {b}: tiered output differs from the resident forward"
        misses += tier.stats()["misses"] - before
        if host is not None:
            ids, _ = qre.route(dev, xs[b])
            host.plan(ids.cpu().reshape(-1).tolist())
            assert tier.state() == host.state(), f"batch {b}: device and host planners disagree"
            assert tier.stats() == host.stats()
    return misses


@pytest.mark.parametrize("case,n_slots", [(c, n) for c in sorted(TIER_CASES) for n in SLOTS[c]])
def test_tier_matches_resident_bitwise(qre, case, n_slots):
    w = synth.scaled(synth.WORKLOADS["tiny"], **TIER_CASES[case])
    say(f"tier case={case} slots={n_slots} E={w.n_experts} k={w.top_k} S={w.S} bits={w.bits}")
    L = synth.make_layer(w)
    dev = to_device(L)
    tier = qre.TieredLayer(to_slow_tier(L, dev), n_slots)
    host = qre.ExpertCache(w.n_experts, n_slots)
    misses = _run_sequence(qre, w, dev, tier, host=host)
    st = tier.stats()
    say(f"  plans={st['plans']} hits={st['hits']} misses={st['misses']} passes={st['passes']}")
    assert st["plans"] == len(ORDER) and misses == st["misses"] > 0
    assert st["resident"] == min(n_slots, st["misses"])
    if n_slots == 1 and w.S * w.top_k > 1:
        assert st["passes"] > 2 * st["plans"]  # chunked: one miss per pass
    slot_of, usage = tier.state()
    assert sum(usage) == st["pairs"]
    tier.close()


def test_tier_against_oracle(qre):
    w = synth.scaled(synth.WORKLOADS["tiny"], **TIER_CASES["long_int4_shared"])
    L = synth.make_layer(w)
    x, _ = gapped_activations(w, L.router_w, L.bias)
    ref = oracle.layer_forward(L, x.numpy())
    dev = to_device(L)
    tier = qre.TieredLayer(to_slow_tier(L, dev), 3)
    out = tier.forward(x.cuda())
    torch.cuda.synchronize()
    assert_close_rms(out.cpu().numpy(), ref["out"], "tier vs oracle")


def test_tier_pinned_hot_set(qre):
    w = synth.scaled(synth.WORKLOADS["tiny"], **TIER_CASES["decode_int4"])
    L = synth.make_layer(w)
    dev = to_device(L)
    tier = qre.TieredLayer(to_slow_tier(L, dev), 10)
    host = qre.ExpertCache(w.n_experts, 10)
    hot = [3, 17, 40, 63, 5, 22]
    _run_sequence(qre, w, dev, tier, order=[7], host=host)  # something resident before the pins
    tier.pin(hot)
    host.pin(hot)
    assert tier.state() == host.state() and tier.stats() == host.stats()
    assert tier.stats()["pinned"] == len(hot)
    _run_sequence(qre, w, dev, tier, order=[0, 1, 2, 3, 4, 0, 5, 1], host=host)
    slot_of, _ = tier.state()
    assert all(slot_of[e] >= 0 for e in hot)
    with pytest.raises(qre.ColibriError):
        tier.pin([0, 1, 2, 4])  # 10 pins would leave no slot for misses
    tier.close()


def test_tier_everything_pinned(qre):
    """All experts pinned: one pass per call, no loads after the pins."""
    w = synth.scaled(synth.WORKLOADS["tiny"], **TIER_CASES["long_int4_shared"])
    L = synth.make_layer(w)
    dev = to_device(L)
    E = w.n_experts
    tier = qre.TieredLayer(to_slow_tier(L, dev), E)
    host = qre.ExpertCache(E, E)
    tier.pin(list(range(E))[::-1])
    host.pin(list(range(E))[::-1])
    _run_sequence(qre, w, dev, tier, order=[0, 1, 2, 0], host=host)
    st = tier.stats()
    assert st["misses"] == 0 and st["passes"] == st["plans"] == 4 and st["pin_loads"] == E
    tier.close()


# every expert pinned, one token, 33 units of I = 2048: the down + combine
# launch does not fuse, so the plan kernel keeps the cache's state
PINNED_UNFUSED = dict(name="tpu", layer="decm", bits=4, hidden=256, inter=2048, n_experts=64, top_k=32, S=1,
                      has_shared=True, var_router=1.0 / 256)


@pytest.mark.parametrize("case", ["decode_int4", "decode_int4_prefetch", "unfused", "unfused_prefetch"])
def test_tier_pinned_after_prefetch(qre, case):
    """Every expert pinned after a prefetch whose loads no plan has consumed:
    the first forward's hits on those slots are late hits (two passes in the
    counters), whether the fused down + combine or the plan kernel keeps the
    state; state and counters follow the host planner's after every batch."""
    kw = PINNED_UNFUSED if case.startswith("unfused") else dict(TIER_CASES["decode_int4"], S=1)
    w = synth.scaled(synth.WORKLOADS["tiny"], **kw)
    say(f"tier pinned case={case} E={w.n_experts} k={w.top_k}")
    L = synth.make_layer(w)
    dev = to_device(L)
    E = w.n_experts
    tier = qre.TieredLayer(to_slow_tier(L, dev), E)
    host = qre.ExpertCache(E, E)
    xs = [synth.activations(w, tag=f"tpin{b}").cuda() for b in range(3)]
    if case.endswith("prefetch"):
        tier.prefetch(xs[0])
        ids_p, _ = qre.route(dev, xs[0])
        host.prefetch(ids_p.cpu().reshape(-1).tolist())
    tier.pin(list(range(E))[::-1])
    host.pin(list(range(E))[::-1])
    for b in [0, 1, 0, 2]:
        got = tier.forward(xs[b])
        ref = qre.moe_layer_forward(dev, xs[b])
        torch.cuda.synchronize()
        assert bits_equal(got, ref), f"batch {b}"
        ids, _ = qre.route(dev, xs[b])
        host.plan(ids.cpu().reshape(-1).tolist())
        assert tier.state() == host.state() and tier.stats() == host.stats(), f"batch {b}"
    st = tier.stats()
    assert st["misses"] == 0 and st["plans"] == 4
    assert st["passes"] == (5 if case.endswith("prefetch") else 4)
    tier.close()


@pytest.mark.parametrize("case", ["decode_int4", "grouped_int4", "small_topp_groups", "many_slots_int2"])
def test_tier_everything_pinned_one_token(qre, case):
    """All experts pinned, one token: the tier runs the resident one-token
    kernels through its slot map (pins in reverse order, so slot != expert);
    outputs equal the resident forward bit for bit and the device planner's
    state the host planner's."""
    w = synth.scaled(synth.WORKLOADS["tiny"], **dict(TIER_CASES[case], S=1))
    L = synth.make_layer(w)
    dev = to_device(L)
    E = w.n_experts
    tier = qre.TieredLayer(to_slow_tier(L, dev), E)
    host = qre.ExpertCache(E, E)
    tier.pin(list(range(E))[::-1])
    host.pin(list(range(E))[::-1])
    _run_sequence(qre, w, dev, tier, order=[0, 1, 2, 0, 3], S=1, host=host)
    st = tier.stats()
    assert st["misses"] == 0 and st["passes"] == st["plans"] == 5 and st["pin_loads"] == E
    tier.close()


def test_tier_device_slow_tier_and_other_width_shared(qre):
    """The slow tier may be device memory; a shared expert at another width
    runs in launches of its own in pass 0."""
    w4 = synth.scaled(synth.WORKLOADS["tiny"], name="tmix4", layer="mix4", bits=4, hidden=512, inter=256,
                      n_experts=32, top_k=4, S=3, has_shared=True, var_router=1.0 / 512)
    w8 = synth.scaled(w4, layer="mix8", bits=8)
    L4, L8 = synth.make_layer(w4), synth.make_layer(w8)
    L = synth.Layer(w4, L4.router_w, L4.bias, L4.gate, L4.up, L4.down, L8.sh_gate, L8.sh_up, L8.sh_down)
    dev = to_device(L)
    for where, n in [("device", 5), ("host", 2)]:
        tier = qre.TieredLayer(to_slow_tier(L, dev, where), n)
        _run_sequence(qre, w4, dev, tier, order=[0, 1, 0, 2])
        for S in (1, 20):
            _run_sequence(qre, w4, dev, tier, order=[5, 6], S=S)
        tier.close()


def test_tier_argument_errors(qre):
    w = synth.scaled(synth.WORKLOADS["tiny"], **TIER_CASES["long_int4_shared"])
    L = synth.make_layer(w)
    dev = to_device(L)
    slow = to_slow_tier(L, dev)
    lib = qre.lib()
    assert lib.colibri_tier_slot_bytes(ctypes.byref(slow.desc), 0) == 0
    assert lib.colibri_tier_slot_bytes(ctypes.byref(slow.desc), w.n_experts + 1) == 0
    nb = lib.colibri_tier_slot_bytes(ctypes.byref(slow.desc), 4)
    mem = torch.empty(nb, dtype=torch.uint8, device="cuda")
    h = ctypes.c_void_p()
    assert lib.colibri_tier_create(ctypes.byref(slow.desc), 4, mem.data_ptr(), nb - 1,
                                   ctypes.byref(h)) == qre.COLI_E_WORKSPACE
    # a routed bank in pageable host memory cannot feed the copy engines
    pageable = np.zeros(L.gate.storage.numel(), dtype=np.uint8)
    desc = qre.LayerDesc.from_buffer_copy(slow.desc)
    desc.gate.data = pageable.ctypes.data
    assert lib.colibri_tier_create(ctypes.byref(desc), 4, mem.data_ptr(), nb,
                                   ctypes.byref(h)) == qre.COLI_E_UNSUPPORTED
    tier = qre.TieredLayer(slow, 4)
    x = synth.activations(w).cuda()
    ws = tier.workspace(w.S)
    with pytest.raises(qre.ColibriError) as ei:
        tier.forward(x, ws=ws[:-256])
    assert ei.value.status == qre.COLI_E_WORKSPACE
    assert tier.stats()["plans"] == 0  # refused before anything ran
    empty = tier.forward(torch.zeros(0, w.hidden, device="cuda"))
    assert empty.shape == (0, w.hidden)
    tier.close()


@pytest.mark.parametrize("all_pinned", [False, True])
def test_tier_forward_in_a_graph(qre, all_pinned):
    """With enough unpinned slots (or every expert pinned: the one-token
    kernels through the slot map) the tiered forward never waits for the
    host, so it can be captured: replays of one captured forward over
    changing inputs equal the resident forward, and the cache state evolves
    as for eager calls."""
    w = synth.scaled(synth.WORKLOADS["tiny"], **TIER_CASES["decode_int4"])
    L = synth.make_layer(w)
    dev = to_device(L)
    n_slots = w.n_experts if all_pinned else 12
    tier = qre.TieredLayer(to_slow_tier(L, dev), n_slots)
    host = qre.ExpertCache(w.n_experts, n_slots)
    if all_pinned:
        tier.pin(list(range(w.n_experts))[::-1])
        host.pin(list(range(w.n_experts))[::-1])
    x_in = torch.zeros(w.S, w.hidden, device="cuda")
    out = torch.zeros_like(x_in)
    ws = tier.workspace(w.S)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tier.forward(x_in, out, ws)
    torch.cuda.synchronize()
    for b in [0, 1, 0, 2, 3, 1]:
        x = synth.activations(w, tag=f"tier{b}").cuda()
        x_in.copy_(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = qre.moe_layer_forward(dev, x)
        torch.cuda.synchronize()
        assert bits_equal(out, ref), f"replay of batch {b}"
        ids, _ = qre.route(dev, x)
        host.plan(ids.cpu().reshape(-1).tolist())
        assert tier.state() == host.state() and tier.stats() == host.stats()
    tier.close()


@pytest.mark.parametrize("n_slots", [16, 40])
def test_tier_prefetch_then_forward(qre, n_slots):
    """Look-ahead prefetches before forwards: outputs stay the resident
    forward's bit for bit, the device state follows the host planner's
    prefetch and plan, and a perfectly predicted batch finds everything
    resident (no misses in its plan)."""
    w = synth.scaled(synth.WORKLOADS["tiny"], **TIER_CASES["decode_int4"])
    L = synth.make_layer(w)
    dev = to_device(L)
    tier = qre.TieredLayer(to_slow_tier(L, dev), n_slots)
    host = qre.ExpertCache(w.n_experts, n_slots)
    xs = [synth.activations(w, tag=f"tier{b}").cuda() for b in range(6)]
    ws = tier.workspace(w.S)
    # (predicted batch, actual batch): right, wrong, two prefetches in a row
    for pred, act in [(0, 0), (1, 2), (3, 3), (4, 1), (5, 5), (2, 2)]:
        tier.prefetch(xs[pred])
        ids_p, _ = qre.route(dev, xs[pred])
        host.prefetch(ids_p.cpu().reshape(-1).tolist())
        if pred == 4:
            tier.prefetch(xs[0])
            ids_p, _ = qre.route(dev, xs[0])
            host.prefetch(ids_p.cpu().reshape(-1).tolist())
        before = tier.stats()["misses"]
        got = tier.forward(xs[act], ws=ws)
        ref = qre.moe_layer_forward(dev, xs[act])
        torch.cuda.synchronize()
        assert bits_equal(got, ref), f"prefetch {pred}, forward {act}"
        ids, _ = qre.route(dev, xs[act])
        host.plan(ids.cpu().reshape(-1).tolist())
        assert tier.state() == host.state() and tier.stats() == host.stats()
        if pred == act:
            assert tier.stats()["misses"] == before, "a perfect prediction leaves no miss"
    assert tier.stats()["prefetches"] == 7
    tier.close()


VERIFY = dict(name="tv4", layer="tv4", bits=4, hidden=512, inter=256, n_experts=32, top_k=4, S=4,
              has_shared=True, rsf=2.5, var_router=1.0 / 512, var_bias=1e-4)


@pytest.mark.parametrize("n_slots", [6, 16])
@pytest.mark.parametrize("lookahead", [False, True])
def test_verify_steps_through_a_stack(qre, n_slots, lookahead):
    """Four verify steps of S = 4 through three tiered layers in one call
    each (colibri_tier_verify_step), with and without the router look-ahead:
    every layer's output equals the resident forward's bit for bit and the
    oracle's layer forward to the output tolerance (after prefetches that
    the look-ahead planned and loaded), and the draft-union statistics equal
    the distinct experts of the oracle's routed ids and their overlap with
    the previous step's.  Layers 0 and 1 share a router and, in steps 0 and
    2, an input, so that the look-ahead predicts layer 1 exactly there.
    Six slots: plans of more than two passes (host round trip); sixteen:
    two passes."""
    n_layers, S = 3, VERIFY["S"]
    w0 = synth.scaled(synth.WORKLOADS["tiny"], **VERIFY)
    Ls = []
    for l in range(n_layers):
        L = synth.make_layer(synth.scaled(w0, layer=f"tv4/l{l}"))
        if l == 1:
            L.router_w, L.bias = Ls[0].router_w, Ls[0].bias
        Ls.append(L)
    devs = [to_device(L) for L in Ls]
    tiers = [qre.TieredLayer(to_slow_tier(L, d), n_slots) for L, d in zip(Ls, devs)]
    E, H, k = w0.n_experts, w0.hidden, w0.top_k
    ws = tiers[0].workspace(S)
    mask = torch.zeros(n_layers, (E + 31) // 32, dtype=torch.int32, device="cuda")
    stats = torch.full((n_layers, 2), -1, dtype=torch.int32, device="cuda")
    out = torch.empty(n_layers, S, H, device="cuda")
    prev = [set() for _ in range(n_layers)]
    for step in range(4):
        xs = []
        for l in range(n_layers):
            if l == 1 and step % 2 == 0:
                xs.append(xs[0].clone())
            else:
                x, _ = gapped_activations(w0, Ls[l].router_w, Ls[l].bias, tag=f"vs{step}/{l}")
                xs.append(x)
        x = torch.stack(xs).contiguous()
        say(f"verify stack: slots={n_slots} lookahead={lookahead} step {step}")
        pf0 = [t.stats()["prefetches"] for t in tiers]
        miss1 = tiers[1].stats()["misses"]
        qre.tier_verify_step(tiers, x.cuda(), out, ws, mask, stats, lookahead=lookahead)
        torch.cuda.synchronize()
        got = out.cpu()
        st = stats.cpu().numpy()
        for l in range(n_layers):
            ref = qre.moe_layer_forward(devs[l], x[l].cuda())
            torch.cuda.synchronize()
            assert bits_equal(out[l], ref), f"step {step} layer {l}: differs from the resident forward"
            r = oracle.layer_forward(Ls[l], x[l].numpy())
            assert_close_rms(got[l].numpy(), r["out"], f"step {step} layer {l} vs oracle")
            union = set(r["ids"].reshape(-1).tolist())
            assert st[l].tolist() == [len(union), len(union & prev[l])], f"step {step} layer {l} statistics"
            prev[l] = union
        pf = [t.stats()["prefetches"] - p for t, p in zip(tiers, pf0)]
        assert pf == ([0, 1, 1] if lookahead else [0, 0, 0])
        if lookahead and step % 2 == 0 and n_slots >= E // 2:
            # layer 1 predicted from its own input, every predicted miss fits
            # the slots: its plan finds all of them resident
            assert tiers[1].stats()["misses"] == miss1, f"step {step}: exact prediction left misses"
    for t in tiers:
        t.close()


def test_verify_step_argument_errors(qre):
    w0 = synth.scaled(synth.WORKLOADS["tiny"], **VERIFY)
    L = synth.make_layer(w0)
    dev = to_device(L)
    t = qre.TieredLayer(to_slow_tier(L, dev), 8)
    S, H = w0.S, w0.hidden
    x = torch.zeros(2, S, H, device="cuda")
    out = torch.empty_like(x)
    ws = t.workspace(S)
    mask = torch.zeros(2, 1, dtype=torch.int32, device="cuda")
    stats = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
    with pytest.raises(qre.ColibriError) as e:
        qre.tier_verify_step([t, t], x, out, ws, mask, stats)  # one tier twice
    assert e.value.status == qre.COLI_E_INVAL
    with pytest.raises(qre.ColibriError) as e:
        qre.tier_verify_step([t], x, out, ws, mask, None)  # statistics need both buffers
    assert e.value.status == qre.COLI_E_INVAL
    with pytest.raises(qre.ColibriError) as e:
        qre.tier_verify_step([t], x, out, ws[:-1].clone())
    assert e.value.status == qre.COLI_E_WORKSPACE
    x9 = torch.zeros(1, 9, H, device="cuda")
    ws9 = t.workspace(9)
    with pytest.raises(qre.ColibriError) as e:
        qre.tier_verify_step([t], x9, torch.empty_like(x9), ws9, lookahead=True)
    assert e.value.status == qre.COLI_E_UNSUPPORTED
    qre.tier_verify_step([t], x9, torch.empty_like(x9), ws9, lookahead=False)
    torch.cuda.synchronize()
    t.close()

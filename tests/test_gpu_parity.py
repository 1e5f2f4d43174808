"""GPU parity at sizes the oracle finishes in seconds: each stage through the
C ABI against the oracle on the same seeded inputs.  Integer results (codes,
ids, dispatch arrays) and the expert outputs y are compared bit for bit;
routing weights and layer outputs within the stated tolerance."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import hand_example
from tests.gpu_common import assert_close_rms, gapped_activations, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qre():
    import quantized_routed_expert_sigmoid_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.lib()
    return m


def test_generator_same_bits_on_cpu_and_gpu(qre):
    key = synth.stream_key("gen-check")
    a = synth.random_bytes(key, 1 << 20, device="cpu")
    b = synth.random_bytes(key, 1 << 20, device="cuda").cpu()
    assert torch.equal(a, b)
    c = synth.random_int8_codes(key, 1 << 18, device="cpu")
    d = synth.random_int8_codes(key, 1 << 18, device="cuda").cpu()
    assert torch.equal(c, d)


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 256), (37, 6144), (5, 2048)])
def test_quantize_q8_0_bit_exact(qre, rows, K):
    say(f"quantize rows={rows} K={K}")
    rng = np.random.default_rng(rows * 1000 + K)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-4, 4, size=(rows, 1))).astype(np.float32)
    x[0, :32] = 0.0                     # an all-zero block
    if K >= 64:
        x[0, 32:64] = np.round(x[0, 32:64])  # integer-valued block
        x[0, 40] = 2.5                  # exact half
    q, d = qre.quantize_q8_0(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    rq, rd = oracle.quantize_q8_0(x)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert d.cpu().numpy().tobytes() == rd.tobytes()


def _small_layer(name, **kw):
    w = synth.scaled(synth.WORKLOADS["tiny"], name=name, **kw)
    return w, synth.make_layer(w)


ROUTE_VARIANTS = {
    "group_limited": dict(name="rv_g", layer="rv_g", n_experts=64, top_k=6, S=37, rsf=2.5, n_group=8,
                          topk_group=3),
    "top_p": dict(name="rv_p", layer="rv_p", n_experts=64, top_k=8, S=37, rsf=2.5, top_p=0.6),
    "group_top_p_small_batch": dict(name="rv_gp", layer="rv_gp", n_experts=64, top_k=8, S=6, rsf=2.5,
                                    n_group=8, topk_group=4, top_p=0.7),
}


@pytest.mark.parametrize("case", sorted(ROUTE_VARIANTS))
def test_route_variant_parity(qre, case):
    """Group-limited selection and adaptive top-p: ids (-1 for dropped slots)
    exact, weights within rtol 2e-6 and exactly 0 for dropped slots."""
    w, L = _small_layer(**ROUTE_VARIANTS[case])
    say(f"route variant {case} S={w.S} E={w.n_experts} k={w.top_k}")
    x, _ = gapped_activations(w, L.router_w, L.bias)
    opts = oracle.route_opts(w.n_group, w.topk_group, w.top_p)
    ids_ref, w_ref, _ = oracle.route(x.numpy(), L.router_w, L.bias, w.top_k, w.rsf, opts)
    ids, wts = qre.route(to_device(L), x.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    got = wts.cpu().numpy()
    assert np.all(got[ids_ref < 0] == 0.0)
    np.testing.assert_allclose(got, w_ref, rtol=2e-6, atol=1e-7)
    if w.top_p < 1.0:
        assert np.any(ids_ref < 0)


def test_dispatch_skips_dropped_slots_bit_exact(qre):
    rng = np.random.default_rng(77)
    S, k, E = 300, 8, 256
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(S)]).astype(np.int32)
    ids[rng.random(ids.shape) < 0.35] = -1
    off, srt, act, na = qre.moe_dispatch(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    ref = oracle.dispatch(ids, E)
    n_pairs = int(ref["offsets"][E])
    assert np.array_equal(off.cpu().numpy(), ref["offsets"])
    assert np.array_equal(srt.cpu().numpy()[:n_pairs], ref["sorted"][:n_pairs])
    n = int(na.cpu()[0])
    assert n == ref["n_active"] and np.array_equal(act.cpu().numpy()[:n], ref["active"])


@pytest.mark.parametrize("case", ["tiny", "odd_experts", "decode_router_s1", "decode_router_s8", "wide_k",
                                  "ragged_tiles", "ragged_tiles_128", "decode_router", "glm_router_s70"])
def test_route_parity(qre, case):
    """Small batches (full-size router rows at 1 and 8 tokens included) take
    the one-workgroup-per-expert router; larger ones the matrix-core router
    with K slices (ragged 64 x 64 tiles, and ragged 128 x 128 tiles over 15
    uneven slices, included)."""
    if case == "tiny":
        w, L = _small_layer("tiny_r")
    elif case == "odd_experts":
        # 20 experts, rows of 328 float4 (not a multiple of 256 threads)
        w, L = _small_layer("odd_e", layer="odd_e", hidden=1312, n_experts=20, top_k=4, S=5, rsf=2.5)
    elif case in ("decode_router_s1", "decode_router_s8"):
        base = synth.WORKLOADS["decode"]
        w = synth.scaled(base, name=f"router_{case[-2:]}", S=int(case[-1]))
        L = synth.Layer(w, synth.router_weights(w), synth.router_bias(w), None, None, None, None, None, None)
    elif case == "wide_k":
        w, L = _small_layer("wide_k", layer="wide_k", n_experts=64, top_k=6, S=37, rsf=2.5)
    elif case == "ragged_tiles":
        w, L = _small_layer("ragged_r", layer="ragged_r", hidden=512, n_experts=100, top_k=6, S=300,
                            rsf=2.5, var_router=1.0 / 512)
    elif case == "ragged_tiles_128":
        # 12 x 3 tiles of 128 (the 64 x 64-wave router), ragged in both
        w, L = _small_layer("ragged_r128", layer="ragged_r128", hidden=256, n_experts=300, top_k=6, S=1500,
                            rsf=2.5, var_router=1.0 / 256)
    elif case == "glm_router_s70":
        base = synth.WORKLOADS["prefill"]
        w = synth.scaled(base, name="router_s70", S=70)
        L = synth.Layer(w, synth.router_weights(w), synth.router_bias(w), None, None, None, None, None, None)
    else:
        base = synth.WORKLOADS["decode"]
        w = synth.scaled(base, name="router_only", S=16)
        L = synth.Layer(w, synth.router_weights(w), synth.router_bias(w), None, None, None, None, None, None)
    say(f"route case={case} S={w.S} E={w.n_experts} k={w.top_k}")
    x, _ = gapped_activations(w, L.router_w, L.bias)
    ids_ref, w_ref, _ = oracle.route(x.numpy(), L.router_w, L.bias, w.top_k, w.rsf)
    # a layer descriptor needs expert banks: give the full-size router small ones
    if L.gate is None:
        wd = synth.scaled(w, name="router_dummy", layer="router_dummy", inter=32, has_shared=False, bits=2)
        D = synth.make_layer(wd)
        L = synth.Layer(wd, L.router_w, L.bias, D.gate, D.up, D.down, None, None, None)
    dev = to_device(L)
    ids, wts = qre.route(dev, x.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(wts.cpu().numpy(), w_ref, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("S,k,E", [(1, 8, 256), (5, 2, 16), (300, 8, 256), (2048, 8, 256), (700, 3, 1000)])
def test_dispatch_bit_exact(qre, S, k, E):
    say(f"dispatch S={S} k={k} E={E}")
    rng = np.random.default_rng(S * 7 + k + E)
    # skewed popularity so some experts get many pairs and some none
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(S)]).astype(np.int32)
    off, srt, act, na = qre.moe_dispatch(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    ref = oracle.dispatch(ids, E)
    assert np.array_equal(off.cpu().numpy(), ref["offsets"])
    assert np.array_equal(srt.cpu().numpy(), ref["sorted"])
    n = int(na.cpu()[0])
    assert n == ref["n_active"]
    assert np.array_equal(act.cpu().numpy()[:n], ref["active"])


def _ffn_case(bits, H, I, E, S, k, seed, g_gu=0, g_d=0):
    rng = np.random.default_rng(seed)
    lo, hi = {8: (-127, 127), 4: (-8, 7), 2: (-2, 1)}[bits]

    def bank(rows, K, group):
        data = np.stack([np.stack([oracle.pack_row(rng.integers(lo, hi + 1, size=K).astype(np.int8), bits)
                                   for _ in range(rows)]) for _ in range(E)])
        ns = rows * (K // group) if group else rows
        scale = (np.abs(rng.standard_normal((E, ns))) * 0.02).astype(np.float32)
        t, s = torch.from_numpy(data), torch.from_numpy(scale)
        return synth.Bank(E, rows, K, bits, [t[i] for i in range(E)], [s[i] for i in range(E)], t, s, group)
    g, u, d = bank(I, H, g_gu), bank(I, H, g_gu), bank(H, I, g_d)
    x = rng.standard_normal((S, H)).astype(np.float32)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(S)]).astype(np.int32)
    return g, u, d, x, ids


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("H,I,E,S,k,scale", [
    (256, 128, 16, 13, 3, 1.0),   # GEMV units (experts with few tokens)
    (96, 64, 4, 9, 2, 1.0),       # ragged 64-row tail of the down projection
    (512, 256, 3, 11, 3, 1.0),    # experts with >= 8 tokens: int8 matrix cores
    (256, 160, 2, 100, 2, 1.0),   # several 32-token MFMA units per expert, ragged N tile
    (96, 96, 5, 40, 3, 1.0),      # MFMA with ragged rows and K tails
    (256, 128, 3, 24, 2, 1e-36),  # tiny activations: block scale * 2^-(8-b) subnormal
    (8192, 64, 4, 6, 2, 1.0),     # K = 8192, few tokens per expert: the octet GEMV (whole-row LDS over 64 KB)
    (2048, 2048, 3, 40, 2, 1.0),  # matrix cores, aligned K loop (whole even step counts per group), two N-tiles
    (2048, 2048, 6, 40, 2, 1.0),  # aligned K loop, one N-tile
    (2048, 2048, 3, 24, 2, 1e-36),  # aligned K loop meets subnormal scale products: the general loop redoes the unit
])
def test_expert_ffn_bit_exact(qre, bits, H, I, E, S, k, scale):
    say(f"ffn bits={bits} H={H} I={I} E={E} S={S} k={k} scale={scale}")
    g, u, d, x, ids = _ffn_case(bits, H, I, E, S, k, seed=bits * 100 + H + S)
    x = (x * np.float32(scale)).astype(np.float32)
    xq, xd = oracle.quantize_q8_0(x)
    disp = oracle.dispatch(ids, E)
    y_ref = np.empty((S * k, H), np.float32)
    G, U, D = oracle.bank(g), oracle.bank(u), oracle.bank(d)
    flat = ids.reshape(-1)
    for pos, p in enumerate(disp["sorted"]):
        y_ref[pos] = oracle.expert_ffn(G, U, D, int(flat[p]), xq[p // k], xd[p // k])["y"]

    def qb(b):
        return qre.QBank(b.storage.cuda(), b.scale_storage.cuda(), bits)
    y = qre.expert_ffn_q(qb(g), qb(u), qb(d), torch.from_numpy(xq).cuda(), torch.from_numpy(xd).cuda(),
                         torch.from_numpy(disp["offsets"]).cuda(), torch.from_numpy(disp["sorted"]).cuda(), k)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert got.tobytes() == y_ref.tobytes(), f"max diff {np.max(np.abs(got - y_ref))}"


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("H,I,E,S,k,g_gu,g_d,scale", [
    (256, 128, 16, 13, 3, 64, 32, 1.0),    # GEMV units
    (96, 64, 4, 9, 2, 32, 64, 1.0),        # ragged down tail; one down group per row
    (512, 256, 3, 11, 3, 128, 256, 1.0),   # matrix cores
    (256, 160, 2, 100, 2, 256, 32, 1.0),   # several MFMA units, ragged N tile
    (96, 96, 5, 40, 3, 32, 96, 1.0),       # MFMA with ragged rows and K tails
    (256, 128, 3, 24, 2, 32, 32, 1e-36),   # tiny activations (subnormal products)
    (512, 512, 2, 40, 2, 32, 32, 1.0),     # aligned matrix-core loop, one scale per block
    (1536, 512, 2, 40, 2, 96, 64, 1.0),    # aligned loop, three blocks per scale (block -> group divide)
])
def test_expert_ffn_grouped_scales_bit_exact(qre, bits, H, I, E, S, k, g_gu, g_d, scale):
    """Group-wise weight scales on both kernel families, y bit for bit."""
    say(f"ffn grouped bits={bits} H={H} I={I} E={E} S={S} k={k} groups={g_gu}/{g_d} scale={scale}")
    g, u, d, x, ids = _ffn_case(bits, H, I, E, S, k, seed=bits * 100 + H + S + 7, g_gu=g_gu, g_d=g_d)
    x = (x * np.float32(scale)).astype(np.float32)
    xq, xd = oracle.quantize_q8_0(x)
    disp = oracle.dispatch(ids, E)
    y_ref = np.empty((S * k, H), np.float32)
    G, U, D = oracle.bank(g), oracle.bank(u), oracle.bank(d)
    flat = ids.reshape(-1)
    for pos, p in enumerate(disp["sorted"]):
        y_ref[pos] = oracle.expert_ffn(G, U, D, int(flat[p]), xq[p // k], xd[p // k])["y"]

    def qb(b):
        return qre.QBank(b.storage.cuda(), b.scale_storage.cuda(), bits, b.group)
    y = qre.expert_ffn_q(qb(g), qb(u), qb(d), torch.from_numpy(xq).cuda(), torch.from_numpy(xd).cuda(),
                         torch.from_numpy(disp["offsets"]).cuda(), torch.from_numpy(disp["sorted"]).cuda(), k)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert got.tobytes() == y_ref.tobytes(), f"max diff {np.max(np.abs(got - y_ref))}"


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("with_shared", [False, True])
def test_hand_two_expert_example(qre, bits, with_shared):
    say(f"hand example bits={bits} shared={with_shared}")
    L = hand_example.layer(bits=bits, with_shared=with_shared)
    x = torch.from_numpy(hand_example.x_values()[None, :])
    out = qre.moe_layer_forward(to_device(L), x.cuda())
    ids, wts = qre.route(to_device(L), x.cuda())
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == [[0, 1]] and wts.cpu().tolist() == [[1.25, 1.25]]
    expect = np.array([float(v) for v in hand_example.out_closed(with_shared)], np.float32)
    assert out.cpu().numpy()[0].tobytes() == expect.tobytes()


SMALL_LAYERS = {
    "tiny": dict(),
    "tiny_shared": dict(name="tiny_sh", has_shared=True, rsf=2.5, top_k=3),
    "tiny_int4_long": dict(name="tiny4", layer="tiny_int4", bits=4, S=37, has_shared=True),
    "tiny_int2_many": dict(name="tiny2", layer="tiny_int2", bits=2, S=64, top_k=4),
    "mid_int4": dict(name="mid4", layer="mid_int4", bits=4, hidden=1024, inter=512, n_experts=32,
                     top_k=4, S=24, has_shared=True, rsf=2.5, var_router=1.0 / 1024, var_bias=1e-4),
    "one_expert": dict(name="one", layer="one", n_experts=4, top_k=1, S=5),
    # 3 tokens x 24 slots: more pairs than one wave places, so the small-batch
    # launch dispatches with the workgroup's counting sort
    "small_many_pairs": dict(name="smp", layer="smp", n_experts=64, top_k=24, S=3, has_shared=True),
    "all_experts": dict(name="all", layer="all", n_experts=8, top_k=8, S=6, has_shared=True),
    # S > 8: experts with >= 8 tokens and the shared expert run on the matrix
    # cores, every expert when the batch has 8 or more pairs per expert
    # (mfma_int4, mfma_int2_long); mfma_int8_mixed mixes both paths
    "mfma_int4": dict(name="mf4", layer="mf4", bits=4, hidden=512, inter=256, n_experts=8, top_k=2,
                      S=64, has_shared=True, rsf=2.5, var_router=1.0 / 512, var_bias=1e-4),
    "mfma_int8_mixed": dict(name="mf8", layer="mf8", bits=8, hidden=256, inter=128, n_experts=32,
                            top_k=4, S=40, has_shared=True),
    "mfma_int2_long": dict(name="mf2", layer="mf2", bits=2, hidden=256, inter=192, n_experts=4,
                           top_k=2, S=150, has_shared=True),
    # the matrix-core threshold's edges: at S = 8 an expert holding all 8
    # tokens stays on the GEMV kernels (two 4-token units); at S = 9 experts
    # with fewer than 8 tokens stay there; with exactly 8 pairs per expert
    # every expert runs on the matrix cores (one with 7 tokens); one pair
    # fewer and the layer mixes both families (8 and 15 tokens on the matrix
    # cores, 6 and 1 on the GEMV kernels)
    "thr_s8_two_experts": dict(name="ts8", layer="ts8", n_experts=2, top_k=1, S=8, has_shared=True),
    "thr_s9": dict(name="ts9", layer="ts9", n_experts=16, top_k=2, S=9),
    "thr_all_mfma": dict(name="tam", layer="tam", bits=4, hidden=512, inter=256, n_experts=4, top_k=2, S=16,
                         has_shared=True, var_router=1.0 / 512),
    "thr_mixed": dict(name="tmx", layer="tam", bits=4, hidden=512, inter=256, n_experts=4, top_k=2, S=15,
                      has_shared=True, var_router=1.0 / 512),
    # one token: selection inside the gate/up kernel, combine inside the down kernel
    "decode_int4": dict(name="dec4", layer="dec4", bits=4, hidden=512, inter=256, n_experts=64, top_k=6,
                        S=1, has_shared=True, rsf=2.5, var_router=1.0 / 512, var_bias=1e-4),
    "decode_int8_noshared": dict(name="dec8", layer="dec8", bits=8, n_experts=32, top_k=4, S=1),
    # H a multiple of 24: the 12-wave down + combine (each CU stages h once)
    "decode_int4_h768": dict(name="dec4w", layer="dec4w", bits=4, hidden=768, inter=256, n_experts=64, top_k=6,
                             S=1, has_shared=True, rsf=2.5, var_router=1.0 / 768, var_bias=1e-4),
    "decode_int2_ragged": dict(name="dec2", layer="dec2", bits=2, hidden=352, inter=96, n_experts=16,
                               top_k=3, S=1, has_shared=True, var_router=1.0 / 352),
    "decode_int4_k2080": dict(name="dec4b", layer="dec4b", bits=4, hidden=2080, inter=160, n_experts=16,
                              top_k=4, S=1, has_shared=True, var_router=1.0 / 2080),
    "decode_int8_k8192": dict(name="dec8b", layer="dec8b", bits=8, hidden=8192, inter=128, n_experts=8,
                              top_k=2, S=1, has_shared=False, var_router=1.0 / 8192),
    # 33 units of I = 2048 do not fit the fused down + combine: separate launches
    "decode_many_slots": dict(name="decm", layer="decm", bits=4, hidden=256, inter=2048, n_experts=64,
                              top_k=32, S=1, has_shared=True, var_router=1.0 / 256),
    # router variants: group-limited selection and adaptive top-p on each path
    "rv_decode_int4": dict(name="rvd", layer="rvd", bits=4, hidden=512, inter=256, n_experts=64, top_k=8,
                           S=1, has_shared=True, rsf=2.5, var_router=1.0 / 512, n_group=8, topk_group=4,
                           top_p=0.6),
    "rv_decode_many_slots": dict(name="rvm", layer="decm", bits=4, hidden=256, inter=2048, n_experts=64,
                                 top_k=32, S=1, has_shared=True, var_router=1.0 / 256, top_p=0.5),
    "rv_small_batch": dict(name="rvs", layer="rvs", bits=8, n_experts=32, top_k=4, S=6, has_shared=True,
                           n_group=4, topk_group=2, top_p=0.8),
    "rv_mfma": dict(name="rvf", layer="rvf", bits=4, hidden=512, inter=256, n_experts=16, top_k=4, S=80,
                    has_shared=True, rsf=2.5, var_router=1.0 / 512, n_group=4, topk_group=2, top_p=0.75),
    # 20 experts and a hidden size (1312) that is not a multiple of 24: the
    # fused down + combine takes its 4-wave workgroups
    "decode_h1312_e20": dict(name="drr", layer="drr", bits=4, hidden=1312, inter=256, n_experts=20, top_k=4,
                             S=1, has_shared=True, rsf=2.5),
    "small_h1312_e20": dict(name="srr", layer="drr", bits=4, hidden=1312, inter=256, n_experts=20, top_k=4,
                            S=5, has_shared=True, rsf=2.5),
    # group-wise weight scales on every path
    "grp_decode_int4": dict(name="gd4", layer="gd4", bits=4, hidden=512, inter=256, n_experts=64, top_k=6,
                            S=1, has_shared=True, rsf=2.5, var_router=1.0 / 512, group=128),
    "grp_decode_many_slots": dict(name="gdm", layer="gdm", bits=4, hidden=256, inter=2048, n_experts=64,
                                  top_k=32, S=1, has_shared=True, var_router=1.0 / 256, group=256),
    "grp_small_int8": dict(name="gs8", layer="gs8", bits=8, n_experts=32, top_k=4, S=6, has_shared=True,
                           group=32),
    "grp_mfma_int2": dict(name="gm2", layer="gm2", bits=2, hidden=256, inter=192, n_experts=4, top_k=2,
                          S=150, has_shared=True, group=64),
    "grp_mfma_int4_topp": dict(name="gmf", layer="gmf", bits=4, hidden=512, inter=256, n_experts=16, top_k=4,
                               S=80, has_shared=True, rsf=2.5, var_router=1.0 / 512, top_p=0.75, group=128),
}


@pytest.mark.parametrize("case", sorted(SMALL_LAYERS))
def test_layer_parity_small(qre, case):
    w = synth.scaled(synth.WORKLOADS["tiny"], **SMALL_LAYERS[case])
    say(f"layer case={case} H={w.hidden} I={w.inter} E={w.n_experts} k={w.top_k} S={w.S} bits={w.bits}")
    L = synth.make_layer(w)
    x, _ = gapped_activations(w, L.router_w, L.bias)
    ref = oracle.layer_forward(L, x.numpy())
    dev = to_device(L)
    ids, _ = qre.route(dev, x.cuda())
    out = qre.moe_layer_forward(dev, x.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_close_rms(out.cpu().numpy(), ref["out"], case)


def _layer_ws_small(w, ws):
    """The dispatch fields of a layer workspace for a batch of at most 8
    tokens, at the offsets the library's workspace layout gives them (fields
    in order, each rounded up to 256 bytes; one logit slice; no matrix-core
    units at this size)."""
    S, E, k, H, I = w.S, w.n_experts, w.top_k, w.hidden, w.inter
    P = S * k
    rows = P + (S if w.has_shared else 0)
    mmin = 9
    per = (mmin - 1 + 3) // 4
    act = min(P, E)
    max_units = min((P + 3 * act) // 4, per * act)
    sizes = [("logits", S * E * 4), ("units", max_units * 16), ("n_units", 16), ("munits", 0),
             ("n_munits", 16), ("hq", rows * I), ("hd", rows * (I // 32) * 4), ("xq", S * H),
             ("xd", S * (H // 32) * 4), ("ids", P * 4), ("w", P * 4), ("offsets", (E + 1) * 4),
             ("sorted", P * 4), ("inv", P * 4), ("active", E * 4), ("n_active", 16)]
    raw = ws.cpu().numpy().view(np.uint8)
    at, f = 0, {}
    for name, n in sizes:
        f[name] = raw[at:at + n]
        at += (n + 255) // 256 * 256
    i32 = {n: f[n].view(np.int32) for n in ("units", "n_units", "ids", "offsets", "sorted", "inv", "active",
                                            "n_active")}
    return i32, max_units


@pytest.mark.parametrize("case,kw", [
    ("tiny_s8_k2", dict(n_experts=16, top_k=2, S=8)),
    ("s4_k8_e64", dict(n_experts=64, top_k=8, S=4, has_shared=True)),
    ("s8_k8_all_fit", dict(n_experts=32, top_k=8, S=8)),
    ("s3_k24_two_waves", dict(n_experts=64, top_k=24, S=3)),
    ("s6_top_p", dict(n_experts=64, top_k=8, S=6, top_p=0.7)),
])
def test_small_batch_dispatch_in_workspace(qre, case, kw):
    """Batches of at most 8 tokens select and dispatch in one launch: up to 64
    pairs are placed directly by one wave, more by the workgroup's counting
    sort.  Either way the dispatch left in the layer workspace is the
    oracle's dispatch of the ids chosen, and the unit lists cover every
    active expert's sorted positions in order, at most 4 per unit."""
    w = synth.scaled(synth.WORKLOADS["tiny"], name="sd_" + case, layer="sd_" + case, **kw)
    say(f"small dispatch case={case} S={w.S} E={w.n_experts} k={w.top_k}")
    L = synth.make_layer(w)
    x, _ = gapped_activations(w, L.router_w, L.bias)
    dev = to_device(L)
    ws = dev.workspace(w.S)
    ws.fill_(0x5A)
    qre.moe_layer_forward(dev, x.cuda(), ws=ws)
    torch.cuda.synchronize()
    f, max_units = _layer_ws_small(w, ws)
    S, k, E = w.S, w.top_k, w.n_experts
    ids = f["ids"][:S * k].reshape(S, k)
    ref_ids = oracle.layer_forward(L, x.numpy())["ids"]
    assert np.array_equal(ids, ref_ids)
    ref = oracle.dispatch(ids, E)
    n_pairs = int(ref["offsets"][E])
    assert np.array_equal(f["offsets"][:E + 1], ref["offsets"])
    assert np.array_equal(f["sorted"][:n_pairs], ref["sorted"][:n_pairs])
    assert np.array_equal(f["inv"][:S * k], ref["inv"])
    n = int(f["n_active"][0])
    assert n == ref["n_active"] and np.array_equal(f["active"][:n], ref["active"])
    want = [(e, int(ref["offsets"][e]) + u, min(4, int(ref["offsets"][e + 1] - ref["offsets"][e]) - u))
            for e in ref["active"] for u in range(0, int(ref["offsets"][e + 1] - ref["offsets"][e]), 4)]
    nu = int(f["n_units"][0])
    assert nu == min(len(want), max_units)
    got = f["units"][:4 * nu].reshape(nu, 4)[:, :3]
    assert np.array_equal(got, np.array(want[:nu], dtype=np.int32).reshape(nu, 3))


@pytest.mark.parametrize("S", [1, 3, 20])
def test_layer_parity_shared_other_bits(qre, S):
    """A shared expert stored at another width runs in launches of its own
    (for one token too, where the fused decode kernels do not apply)."""
    w4 = synth.scaled(synth.WORKLOADS["tiny"], name="mix4", layer="mix4", bits=4, hidden=512, inter=256,
                      n_experts=32, top_k=4, S=S, has_shared=True, var_router=1.0 / 512)
    w8 = synth.scaled(w4, layer="mix8", bits=8)
    L4, L8 = synth.make_layer(w4), synth.make_layer(w8)
    L = synth.Layer(w4, L4.router_w, L4.bias, L4.gate, L4.up, L4.down, L8.sh_gate, L8.sh_up, L8.sh_down)
    say(f"layer shared int8 / routed int4 S={S}")
    x, _ = gapped_activations(w4, L.router_w, L.bias)
    ref = oracle.layer_forward(L, x.numpy())
    out = qre.moe_layer_forward(to_device(L), x.cuda())
    torch.cuda.synchronize()
    assert_close_rms(out.cpu().numpy(), ref["out"], f"mixed S={S}")


def test_layer_empty_batch_is_noop(qre):
    w, L = _small_layer("tiny_e")
    dev = to_device(L)
    x = torch.zeros(0, w.hidden, device="cuda")
    out = qre.moe_layer_forward(dev, x)
    torch.cuda.synchronize()
    assert out.shape == (0, w.hidden)


@pytest.mark.parametrize("case", ["tiny_int4_long", "decode_int4"])
def test_layer_repeatable_bitwise(qre, case):
    """Two runs on the same inputs give identical bits (no atomics on data)."""
    w = synth.scaled(synth.WORKLOADS["tiny"], **SMALL_LAYERS[case])
    L = synth.make_layer(w)
    dev = to_device(L)
    x = synth.activations(w).cuda()
    a = qre.moe_layer_forward(dev, x).cpu()
    b = qre.moe_layer_forward(dev, x).cpu()
    assert torch.equal(a, b)


@pytest.mark.parametrize("case", ["decode_int4", "decode_int2_ragged", "decode_int4_k2080", "decode_int8_noshared",
                                  "decode_int4_h768", "decode_h1312_e20"])
def test_decode_path_matches_small_batch_bitwise(qre, case):
    """One token through the fused decode launches (selection inside gate/up,
    the shared expert as one-wave jobs, combine inside down) gives the same
    bits as that token twice in a two-token batch (the small-batch kernels):
    one canonical fold and one Q8_0 of h on every path."""
    w = synth.scaled(synth.WORKLOADS["tiny"], **SMALL_LAYERS[case])
    L = synth.make_layer(w)
    x, _ = gapped_activations(w, L.router_w, L.bias)
    say(f"decode vs two-token batch case={case}")
    dev = to_device(L)
    x1 = x[:1].contiguous()
    x2 = torch.cat([x1, x1]).contiguous()
    out1 = qre.moe_layer_forward(dev, x1.cuda()).cpu()
    out2 = qre.moe_layer_forward(dev, x2.cuda()).cpu()
    assert torch.equal(out1[0], out2[0]) and torch.equal(out1[0], out2[1]), \
        f"max diff {(out1[0] - out2[0]).abs().max().item()}"

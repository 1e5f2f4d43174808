"""Host-side checks of the GPU library that need no GPU: the container
unpacking logic of its kernels (compiled for the CPU against emulated
instructions) versus the oracle, and the C ABI's exports and argument
validation (every error path returns before any HIP call)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HARNESS_SRC = os.path.join(ROOT, "tests", "qdot_harness.cpp")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("harness") / "libqdot_harness.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-o", out, HARNESS_SRC], check=True)
    lib = ctypes.CDLL(out)
    for fn in (lib.harness_block_partial, lib.harness_block_dot):
        fn.restype = ctypes.c_int32
        fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("form", ["block_partial", "block_dot"])
@pytest.mark.parametrize("bits,lo,hi", [(8, -127, 127), (4, -8, 7), (2, -2, 1)])
def test_kernel_unpack_matches_oracle_partials(harness, bits, lo, hi, form):
    """Both kernel forms of the exact block partial (the matrix-core operand
    order and the VALU form, int4 by nibble dot products) against the
    oracle's, on random codes and the extremes of both ranges: activation
    codes of +-127 and 120..127 (where a plain two-nibble split of the code
    would overflow)."""
    fn = getattr(harness, "harness_" + form)
    rng = np.random.default_rng(7 + bits)
    K = 32 * 64
    for trial in range(10):
        codes = rng.integers(lo, hi + 1, size=K).astype(np.int8)
        if trial == 0:
            codes[:] = lo  # extreme values
        if trial in (1, 8):
            codes[:] = hi
        row = oracle.pack_row(codes, bits)
        q = rng.integers(-127, 128, size=K).astype(np.int8)
        if trial == 2:
            q[:] = -127
        if trial in (3, 8):
            q[:] = 127
        if trial == 9:
            q = rng.integers(120, 128, size=K).astype(np.int8) * rng.choice(np.array([-1, 1], np.int8), size=K)
        bb = 4 * bits  # bytes per 32-element block
        for b in range(K // 32):
            wblk = np.ascontiguousarray(row[b * bb:(b + 1) * bb])
            qb = np.ascontiguousarray(q[32 * b:32 * (b + 1)])
            got = fn(bits, wblk.ctypes.data, qb.ctypes.data)
            assert got == oracle.block_partial(row, bits, q, b), (trial, b)


# ---------------------------------------------------------------------------
# C ABI: exports and validation (no kernel is launched by any call below)
# ---------------------------------------------------------------------------

def _declared_symbols():
    with open(os.path.join(ROOT, "include", "colibri.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(colibri_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def capi():
    import quantized_routed_expert_sigmoid_amd as qre
    return qre


def test_library_exports_every_declared_symbol(capi):
    lib = capi.lib()
    syms = _declared_symbols()
    assert len(syms) == 28
    for name in syms:
        assert hasattr(lib, name), name


def test_status_strings(capi):
    for code in range(6):
        assert capi.status_string(code)
    assert capi.status_string(99) == "unknown status"


def _fake_layer(capi, **over):
    """A descriptor with plausible (fake, never dereferenced) device pointers."""
    H, I, E, k = 256, 128, 16, 2
    fake = 0x10000000

    def bank(n, rows, K, q=8):
        return capi.QBankDesc(fake, fake, n, rows, K, q)
    d = dict(hidden=H, inter=I, n_experts=E, top_k=k, rsf=1.0, router_w=fake, router_bias=fake,
             gate=bank(E, I, H), up=bank(E, I, H), down=bank(E, H, I), has_shared=1,
             sh_gate=bank(1, I, H), sh_up=bank(1, I, H), sh_down=bank(1, H, I))
    d.update(n_group=1, topk_group=1, top_p=1.0)
    d.update(over)
    return capi.LayerDesc(d["hidden"], d["inter"], d["n_experts"], d["top_k"], d["rsf"],
                          d["router_w"], d["router_bias"], d["gate"], d["up"], d["down"],
                          d["has_shared"], d["sh_gate"], d["sh_up"], d["sh_down"],
                          d["n_group"], d["topk_group"], d["top_p"])


def test_tier_sizes_and_validation_before_any_hip_call(capi):
    """Slot-bank sizes and the tier calls' argument checks (none of them
    reaches the HIP runtime)."""
    lib = capi.lib()
    L = _fake_layer(capi, gate=capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 256, 4),
                    up=capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 256, 4),
                    down=capi.QBankDesc(0x10000000, 0x10000000, 16, 256, 128, 2))
    n3 = lib.colibri_tier_slot_bytes(ctypes.byref(L), 3)
    n5 = lib.colibri_tier_slot_bytes(ctypes.byref(L), 5)
    # per slot: gate + up 128 rows * 128 B and 128 scales each; down 256 rows * 32 B and 256 scales
    per_slot = 2 * (128 * 128 + 128 * 4) + 256 * 32 + 256 * 4
    assert n3 >= 3 * per_slot and n3 % 256 == 0
    assert n5 - n3 == 2 * per_slot  # the state regions of 3 and 5 slots round to the same 256 B
    assert lib.colibri_tier_slot_bytes(ctypes.byref(L), 0) == 0
    assert lib.colibri_tier_slot_bytes(ctypes.byref(L), 17) == 0
    h = ctypes.c_void_p()
    assert lib.colibri_tier_create(ctypes.byref(L), 3, 0x10000000, n3, None) == capi.COLI_E_INVAL
    assert lib.colibri_tier_create(ctypes.byref(L), 0, 0x10000000, n3, ctypes.byref(h)) == capi.COLI_E_INVAL
    assert lib.colibri_tier_create(ctypes.byref(L), 3, None, n3, ctypes.byref(h)) == capi.COLI_E_INVAL
    assert lib.colibri_tier_create(ctypes.byref(L), 3, 0x10000010, n3,
                                   ctypes.byref(h)) == capi.COLI_E_UNSUPPORTED
    assert lib.colibri_tier_create(ctypes.byref(L), 3, 0x10000000, n3 - 1,
                                   ctypes.byref(h)) == capi.COLI_E_WORKSPACE
    Lb = _fake_layer(capi, top_k=0)
    assert lib.colibri_tier_create(ctypes.byref(Lb), 3, 0x10000000, n3, ctypes.byref(h)) == capi.COLI_E_INVAL
    assert not h.value
    assert lib.colibri_tier_forward(None, 0x10000000, 1, 0x10000000, 0x10000000, 1 << 20,
                                    None) == capi.COLI_E_INVAL
    assert lib.colibri_tier_pin(None, None, 0, None) == capi.COLI_E_INVAL
    # the verify step: no tier array, no layers, a null tier in the array
    f = 0x10000000
    assert lib.colibri_tier_verify_step(None, 2, f, 4, f, 1, f, 1 << 20, f, f, None) == capi.COLI_E_INVAL
    one = (ctypes.c_void_p * 1)(None)
    assert lib.colibri_tier_verify_step(one, 0, f, 4, f, 1, f, 1 << 20, f, f, None) == capi.COLI_E_INVAL
    assert lib.colibri_tier_verify_step(one, 1, f, 4, f, 1, f, 1 << 20, f, f, None) == capi.COLI_E_INVAL
    assert lib.colibri_tier_workspace_bytes(None, 4) == 0
    st = capi.CacheStats()
    assert lib.colibri_tier_stats(None, ctypes.byref(st), None) == capi.COLI_E_INVAL
    assert lib.colibri_tier_state(None, None, None, None) == capi.COLI_E_INVAL
    lib.colibri_tier_destroy(None)


def test_group_wise_scale_validation(capi):
    lib = capi.lib()
    f = 0x10000000

    def qb(n, rows, K, q=4, group=0):
        return capi.QBankDesc(f, f, n, rows, K, q, group)
    ok = _fake_layer(capi, gate=qb(16, 128, 256, group=128), up=qb(16, 128, 256, group=128),
                     down=qb(16, 256, 128, group=32))
    assert lib.colibri_workspace_bytes(ctypes.byref(ok), 4) > 0
    for bad in (dict(gate=qb(16, 128, 256, group=48), up=qb(16, 128, 256, group=48)),   # not a multiple of 32
                dict(gate=qb(16, 128, 256, group=96), up=qb(16, 128, 256, group=96)),   # does not divide K
                dict(down=qb(16, 256, 128, group=-32)),
                dict(gate=qb(16, 128, 256, group=512), up=qb(16, 128, 256, group=512))):  # larger than K
        assert lib.colibri_workspace_bytes(ctypes.byref(_fake_layer(capi, **bad)), 4) == 0
    # gate and up must share the group size (as they share the width)
    mixed = _fake_layer(capi, gate=qb(16, 128, 256, group=64), up=qb(16, 128, 256, group=128))
    assert lib.colibri_workspace_bytes(ctypes.byref(mixed), 4) == 0


def test_workspace_size_and_invalid_layers(capi):
    lib = capi.lib()
    L = _fake_layer(capi)
    n8 = lib.colibri_workspace_bytes(ctypes.byref(L), 8)
    n1 = lib.colibri_workspace_bytes(ctypes.byref(L), 1)
    assert n8 > n1 > 0 and n8 % 256 == 0
    for bad in (dict(hidden=250), dict(inter=0), dict(top_k=17), dict(top_k=0), dict(n_experts=0),
                dict(router_w=0), dict(gate=capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 255, 8)),
                dict(gate=capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 256, 3)),
                dict(gate=capi.QBankDesc(0x10000008, 0x10000000, 16, 128, 256, 8)),
                dict(down=capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 128, 4)),
                dict(sh_down=capi.QBankDesc(0x10000000, 0x10000000, 2, 256, 128, 8))):
        Lb = _fake_layer(capi, **bad)
        assert lib.colibri_workspace_bytes(ctypes.byref(Lb), 8) == 0, bad
    assert lib.colibri_workspace_bytes(None, 8) == 0
    assert lib.colibri_workspace_bytes(ctypes.byref(L), -1) == 0


def test_router_variant_validation(capi):
    lib = capi.lib()
    ok = [dict(n_group=0), dict(n_group=4, topk_group=2), dict(n_group=8, topk_group=1, top_k=2),
          dict(top_p=0.0), dict(top_p=0.5), dict(top_p=1.0), dict(top_p=3.0),
          dict(n_group=4, topk_group=4, top_p=0.7)]
    for good in ok:
        assert lib.colibri_workspace_bytes(ctypes.byref(_fake_layer(capi, **good)), 8) > 0, good
    # E = 16: groups must divide it, hold >= 2 experts each, and keep >= top_k experts
    bad = [dict(n_group=3, topk_group=1), dict(n_group=16, topk_group=4), dict(n_group=4, topk_group=0),
           dict(n_group=4, topk_group=5), dict(n_group=8, topk_group=1, top_k=3), dict(n_group=-1),
           dict(top_p=-0.5), dict(top_p=float("nan"))]
    for b in bad:
        assert lib.colibri_workspace_bytes(ctypes.byref(_fake_layer(capi, **b)), 8) == 0, b


def test_layer_forward_error_paths(capi):
    lib = capi.lib()
    L = _fake_layer(capi)
    fake = 0x20000000
    need = lib.colibri_workspace_bytes(ctypes.byref(L), 8)
    f = lib.colibri_moe_layer_forward
    assert f(None, fake, 8, fake, fake, need, None) == capi.COLI_E_INVAL
    assert f(ctypes.byref(L), fake, -1, fake, fake, need, None) == capi.COLI_E_INVAL
    assert f(ctypes.byref(L), fake, 0, fake, fake, need, None) == capi.COLI_OK  # empty batch: no-op
    assert f(ctypes.byref(L), None, 8, fake, fake, need, None) == capi.COLI_E_INVAL
    assert f(ctypes.byref(L), fake, 8, None, fake, need, None) == capi.COLI_E_INVAL
    assert f(ctypes.byref(L), fake, 8, fake, None, need, None) == capi.COLI_E_INVAL
    assert f(ctypes.byref(L), fake + 4, 8, fake, fake, need, None) == capi.COLI_E_UNSUPPORTED
    assert f(ctypes.byref(L), fake, 8, fake, fake + 16, need, None) == capi.COLI_E_UNSUPPORTED
    assert f(ctypes.byref(L), fake, 8, fake, fake, need - 1, None) == capi.COLI_E_WORKSPACE
    assert f(ctypes.byref(L), fake, 70000, fake, fake, 1 << 40, None) == capi.COLI_E_UNSUPPORTED
    Lq = _fake_layer(capi, up=capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 256, 4))
    assert f(ctypes.byref(Lq), fake, 8, fake, fake, need, None) == capi.COLI_E_UNSUPPORTED
    Lk = _fake_layer(capi, top_k=65, n_experts=100,
                     gate=capi.QBankDesc(0x10000000, 0x10000000, 100, 128, 256, 8))
    assert f(ctypes.byref(Lk), fake, 8, fake, fake, need, None) == capi.COLI_E_UNSUPPORTED


def test_stage_calls_error_paths(capi):
    lib = capi.lib()
    L = _fake_layer(capi)
    fake = 0x20000000
    need = lib.colibri_workspace_bytes(ctypes.byref(L), 4)
    assert lib.colibri_quantize_q8_0(fake, 4, 250, fake, fake, None) == capi.COLI_E_INVAL
    assert lib.colibri_quantize_q8_0(fake, -1, 256, fake, fake, None) == capi.COLI_E_INVAL
    assert lib.colibri_quantize_q8_0(fake, 0, 256, fake, fake, None) == capi.COLI_OK
    assert lib.colibri_quantize_q8_0(None, 4, 256, fake, fake, None) == capi.COLI_E_INVAL
    assert lib.colibri_quantize_q8_0(fake + 8, 4, 256, fake, fake, None) == capi.COLI_E_UNSUPPORTED
    assert lib.colibri_route(ctypes.byref(L), fake, 4, None, fake, fake, need, None) == capi.COLI_E_INVAL
    assert lib.colibri_route(ctypes.byref(L), fake, 4, fake, fake, fake, need - 256, None) == capi.COLI_E_WORKSPACE
    assert lib.colibri_route(ctypes.byref(L), fake, 0, fake, fake, fake, 0, None) == capi.COLI_OK
    d = lib.colibri_moe_dispatch
    assert d(fake, 4, 3, 2, fake, fake, fake, fake, None, 0, None) == capi.COLI_E_INVAL  # k > E
    assert d(fake, 4, 2, 2000, fake, fake, fake, fake, None, 0, None) == capi.COLI_E_UNSUPPORTED
    assert d(fake, 4, 2, 16, None, fake, fake, fake, None, 0, None) == capi.COLI_E_INVAL
    assert d(fake, -2, 2, 16, fake, fake, fake, fake, None, 0, None) == capi.COLI_E_INVAL
    g = capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 256, 8)
    dn = capi.QBankDesc(0x10000000, 0x10000000, 16, 256, 128, 8)
    wsz = lib.colibri_expert_ffn_workspace_bytes(ctypes.byref(g), ctypes.byref(dn), 4, 2)
    assert wsz > 0
    ffn = lib.colibri_expert_ffn_q
    args = [ctypes.byref(g), ctypes.byref(g), ctypes.byref(dn), fake, fake, 4, fake, fake, 2, fake, fake]
    assert ffn(*args, wsz - 1, None) == capi.COLI_E_WORKSPACE
    bad_up = capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 256, 2)
    assert ffn(ctypes.byref(g), ctypes.byref(bad_up), ctypes.byref(dn), *args[3:], wsz, None) == capi.COLI_E_UNSUPPORTED
    bad_dn = capi.QBankDesc(0x10000000, 0x10000000, 16, 128, 128, 8)
    assert ffn(ctypes.byref(g), ctypes.byref(g), ctypes.byref(bad_dn), *args[3:], wsz, None) == capi.COLI_E_INVAL
    assert ffn(*args[:9], None, fake, wsz, None) == capi.COLI_E_INVAL

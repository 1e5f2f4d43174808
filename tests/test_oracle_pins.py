"""Pins of the oracle against facts that do not come from the oracle itself:
the pages' stated layouts and invariants, closed forms, brute force on tiny
inputs, error bounds and special cases.  CPU only."""

import json
import math
import pathlib
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import hand_example

RNG = np.random.default_rng(12345)
GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"
U = 2.0 ** -24  # fp32 unit roundoff


def ulp32(v):
    v = np.abs(np.float32(v))
    return float(np.spacing(v)) if v != 0 else float(np.finfo(np.float32).smallest_subnormal)


# ---------------------------------------------------------------------------
# Q8_0 activation quantisation (README, integer dot-product item)
# ---------------------------------------------------------------------------

def _blocks(n_blocks, scale_spread=True):
    v = RNG.standard_normal((n_blocks, 32)).astype(np.float32)
    if scale_spread:
        v *= (10.0 ** RNG.uniform(-6, 6, size=(n_blocks, 1))).astype(np.float32)
    return v


def test_q8_0_brute_force_nearest_code():
    v = _blocks(400)
    q, d = oracle.quantize_q8_0(v.reshape(-1))
    q, d = q.reshape(400, 32), d.reshape(400)
    for b in range(400):
        amax = float(np.max(np.abs(v[b].astype(np.float64))))
        # scale: amax / 127 correctly rounded to fp32
        assert abs(float(d[b]) - amax / 127.0) <= 0.5 * ulp32(d[b])
        # every code is the nearest of the 255 codes to v / d (ties within
        # fp32 rounding of v * (1/d) may go either way)
        codes = np.arange(-127, 128, dtype=np.float64)
        for i in range(32):
            t = float(v[b, i]) / float(d[b])
            best = codes[np.argmin(np.abs(codes - t))]
            if abs(abs(t - math.floor(t)) - 0.5) > 1e-5:
                assert q[b, i] == best, (b, i, t)
        # the element of largest magnitude maps to +-127
        i_max = int(np.argmax(np.abs(v[b])))
        assert abs(int(q[b, i_max])) == 127


def test_q8_0_special_cases():
    # all-zero block: scale 0, codes 0
    q, d = oracle.quantize_q8_0(np.zeros(32, np.float32))
    assert d[0] == 0.0 and not q.any()
    # integer block with amax 127 is its own encoding (scale exactly 1)
    ints = RNG.integers(-127, 128, size=64).astype(np.float32)
    ints[0], ints[40] = 127, -127
    q_ints, d = oracle.quantize_q8_0(ints)
    assert np.all(d == 1.0) and np.array_equal(q_ints.astype(np.float32), ints)
    # halves round away from zero (banker's rounding would give 2 and -2)
    v = np.zeros(32, np.float32)
    v[0], v[1], v[2], v[3] = 127, 2.5, -2.5, 0.5
    q, d = oracle.quantize_q8_0(v)
    assert (q[1], q[2], q[3]) == (3, -3, 1)
    assert oracle.round_half_away(-0.5) == -1.0 and oracle.round_half_away(0.49999997) == 0.0
    # blocks are independent: a huge value in block 1 leaves block 0 alone
    v = np.concatenate([ints[:32], np.full(32, 1e6, np.float32)])
    q2, d2 = oracle.quantize_q8_0(v)
    assert d2[0] == 1.0 and np.array_equal(q2[:32], q_ints[:32])


def test_q8_0_reconstruction_bound():
    v = _blocks(200).reshape(-1)
    q, d = oracle.quantize_q8_0(v)
    rec = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32)
    err = np.abs(rec - v.astype(np.float64))
    assert np.all(err <= np.repeat(d.astype(np.float64), 32) * (0.5 + 1e-5))


# ---------------------------------------------------------------------------
# Weight containers (deep dive 5.1: two int4 per byte, first element in the
# high nibble; README: packing bit-identical to the int8 container)
# ---------------------------------------------------------------------------

def test_container_hand_bytes():
    row4 = np.array([0x7F, 0x80, 0x1E], np.uint8)
    assert [oracle.weight_code(row4, 4, c) for c in range(6)] == [7, -1, -8, 0, 1, -2]
    row2 = np.array([0b01101100], np.uint8)
    assert [oracle.weight_code(row2, 2, c) for c in range(4)] == [1, -2, -1, 0]
    row8 = np.array([0xFF, 0x81, 0x7F, 0x00], np.uint8)
    assert [oracle.weight_code(row8, 8, c) for c in range(4)] == [-1, -127, 127, 0]
    assert list(oracle.pack_row(np.array([7, -1, -8, 0, 1, -2], np.int8), 4)) == [0x7F, 0x80, 0x1E]
    assert list(oracle.pack_row(np.array([1, -2, -1, 0], np.int8), 2)) == [0b01101100]


@pytest.mark.parametrize("bits,lo,hi", [(8, -128, 127), (4, -8, 7), (2, -2, 1)])
def test_container_round_trip(bits, lo, hi):
    codes = RNG.integers(lo, hi + 1, size=256).astype(np.int8)
    row = oracle.pack_row(codes, bits)
    assert row.size == 256 * bits // 8
    assert np.array_equal(oracle.unpack_row(row, bits, 256), codes)


@pytest.mark.parametrize("bits,lo,hi", [(4, -8, 7), (2, -2, 1)])
def test_packed_equals_int8_container(bits, lo, hi):
    K = 256
    codes = RNG.integers(lo, hi + 1, size=K).astype(np.int8)
    packed, as8 = oracle.pack_row(codes, bits), oracle.pack_row(codes, 8)
    x = RNG.standard_normal(K).astype(np.float32)
    q, d = oracle.quantize_q8_0(x)
    for b in range(K // 32):
        assert oracle.block_partial(packed, bits, q, b) == oracle.block_partial(as8, 8, q, b)
    a = np.float32(oracle.qdot(packed, bits, 0.37, q, d))
    c = np.float32(oracle.qdot(as8, 8, 0.37, q, d))
    assert a.tobytes() == c.tobytes()


# ---------------------------------------------------------------------------
# Integer dot path: block partials and the fold
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits,lo,hi", [(8, -127, 127), (4, -8, 7), (2, -2, 1)])
def test_block_partials_brute_force(bits, lo, hi):
    K = 192
    codes = RNG.integers(lo, hi + 1, size=K).astype(np.int64)
    row = oracle.pack_row(codes.astype(np.int8), bits)
    q = RNG.integers(-127, 128, size=K).astype(np.int64)
    total = 0
    for b in range(K // 32):
        s = oracle.block_partial(row, bits, q.astype(np.int8), b)
        brute = sum(int(codes[32 * b + i]) * int(q[32 * b + i]) for i in range(32))
        assert s == brute
        total += s
    assert total == int(np.dot(codes, q))
    # all weights 1: the partial is the block's code sum
    ones = oracle.pack_row(np.ones(K, np.int8), bits)
    assert oracle.block_partial(ones, bits, q.astype(np.int8), 2) == int(q[64:96].sum())


@pytest.mark.parametrize("bits,lo,hi", [(8, -127, 127), (4, -8, 7), (2, -2, 1)])
def test_fold_error_bound(bits, lo, hi):
    K = 6144
    for trial in range(20):
        codes = RNG.integers(lo, hi + 1, size=K).astype(np.int8)
        row = oracle.pack_row(codes, bits)
        x = RNG.standard_normal(K).astype(np.float32) * np.float32(10.0 ** RNG.uniform(-3, 3))
        q, d = oracle.quantize_q8_0(x)
        scale = np.float32(abs(RNG.standard_normal()) * 0.02)
        got = float(oracle.qdot(row, bits, float(scale), q, d))
        exact = oracle.qdot_f64(row, bits, float(scale), q, d)
        parts = np.array([oracle.block_partial(row, bits, q, b) for b in range(K // 32)], np.float64)
        n = K // 32 + 1
        bound = (n * U / (1 - n * U)) * float(scale) * float(np.sum(np.abs(d.astype(np.float64) * parts)))
        assert abs(got - exact) <= bound + 1e-30, (trial, got, exact, bound)


def test_fold_exact_on_integers():
    K = 128
    codes = RNG.integers(-127, 128, size=K).astype(np.int8)
    row = oracle.pack_row(codes, 8)
    q = RNG.integers(-127, 128, size=K).astype(np.int8)
    d = np.ones(K // 32, np.float32)
    assert oracle.qdot(row, 8, 1.0, q, d) == float(np.dot(codes.astype(np.int64), q.astype(np.int64)))
    # scales enter per block: doubling block 3's scale adds its partial once more
    d2 = d.copy()
    d2[3] = 2.0
    p3 = oracle.block_partial(row, 8, q, 3)
    assert oracle.qdot(row, 8, 1.0, q, d2) == oracle.qdot(row, 8, 1.0, q, d) + p3
    # the row scale multiplies the folded sum
    assert oracle.qdot(row, 8, 0.5, q, d) == 0.5 * oracle.qdot(row, 8, 1.0, q, d)


def _fold_fixture_case(case, bits):
    """Row, codes and block scales of a tests/golden/fold_order.json case."""
    w_cols, q_cols = [], []
    for blk in case["blocks"]:
        w_cols += [blk["w"]] * 32
        c = blk["codes"]
        q_cols += [int(c.split()[1])] * 32 if isinstance(c, str) else list(c)
    codes = np.array(w_cols, np.int8)
    q = np.array(q_cols, np.int8)
    d = np.array([blk["d"] for blk in case["blocks"]], np.float32)
    # the fixture's scales are fp32 numbers as written
    assert [float(v) for v in d] == [blk["d"] for blk in case["blocks"]]
    return oracle.pack_row(codes, bits), q, d


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_fold_order_hand_worked(bits):
    """The fold is one ascending chain of fused multiply-adds from +0: two
    hand-worked rows (tests/golden/fold_order.json) whose exact results
    differ from a fold in four block groups, from a descending chain and
    from rounding each product before the add."""
    fx = json.loads((GOLDEN / "fold_order.json").read_text())
    for case in fx["cases"]:
        row, q, d = _fold_fixture_case(case, bits)
        assert len(q) == case["K"]
        parts = [oracle.block_partial(row, bits, q, b) for b in range(case["K"] // 32)]
        assert parts == case["partials"]
        got = oracle.qdot(row, bits, case["row_scale"], q, d)
        assert got == case["expected"], (case["name"], got)
        assert case["expected"] != case["expected_if_grouped_in_fours"]
        gs = case["group_scales"]
        s = np.array(gs["scales"], np.float32)
        got_g = oracle.qdot_grouped(row, bits, s, gs["group"], q, d)
        assert got_g == gs["expected"], (case["name"], got_g)


# ---------------------------------------------------------------------------
# group-wise weight scales (one scale per `group` columns of a row)

GROUP_CASES = [(8, -127, 127, 32), (4, -8, 7, 128), (2, -2, 1, 256), (4, -8, 7, 64)]


@pytest.mark.parametrize("bits,lo,hi,group", GROUP_CASES)
def test_grouped_unit_and_power_of_two_scales(bits, lo, hi, group):
    """All group scales 1: exactly the per-row fold with row scale 1.  All
    equal to 2^j: every product and partial sum is scaled exactly, so the
    result is 2^j times it, bit for bit."""
    K = 1024
    for trial in range(10):
        codes = RNG.integers(lo, hi + 1, size=K).astype(np.int8)
        row = oracle.pack_row(codes, bits)
        x = RNG.standard_normal(K).astype(np.float32) * np.float32(10.0 ** RNG.uniform(-2, 2))
        q, d = oracle.quantize_q8_0(x)
        base = np.float32(oracle.qdot(row, bits, 1.0, q, d))
        ones = np.ones(K // group, np.float32)
        assert np.float32(oracle.qdot_grouped(row, bits, ones, group, q, d)) == base
        for j in (-3, 5):
            s = np.full(K // group, 2.0 ** j, np.float32)
            assert np.float32(oracle.qdot_grouped(row, bits, s, group, q, d)) == np.float32(base * 2.0 ** j)


@pytest.mark.parametrize("bits,lo,hi,group", GROUP_CASES)
def test_grouped_scale_reaches_only_its_columns(bits, lo, hi, group):
    """Scale 1 on group g0 and 0 elsewhere equals the per-row fold of the row
    with every code outside columns [g0*group, (g0+1)*group) set to zero (a
    wrong group index, a scale applied per block instead of per group, or a
    leftover row scale all break this)."""
    K = 1024
    for g0 in range(K // group):
        codes = RNG.integers(lo, hi + 1, size=K).astype(np.int8)
        row = oracle.pack_row(codes, bits)
        x = RNG.standard_normal(K).astype(np.float32)
        q, d = oracle.quantize_q8_0(x)
        s = np.zeros(K // group, np.float32)
        s[g0] = 1.0
        masked = codes.copy()
        keep = np.zeros(K, bool)
        keep[g0 * group:(g0 + 1) * group] = True
        masked[~keep] = 0
        want = np.float32(oracle.qdot(oracle.pack_row(masked, bits), bits, 1.0, q, d))
        assert np.float32(oracle.qdot_grouped(row, bits, s, group, q, d)) == want


@pytest.mark.parametrize("bits,lo,hi,group", GROUP_CASES)
def test_grouped_fold_error_bound(bits, lo, hi, group):
    """Against the unblocked fp64 sum of s[c / group] * code * q * d: within
    the fold's bound plus one rounding of each coefficient."""
    K = 6144
    for trial in range(10):
        codes = RNG.integers(lo, hi + 1, size=K).astype(np.int8)
        row = oracle.pack_row(codes, bits)
        x = RNG.standard_normal(K).astype(np.float32) * np.float32(10.0 ** RNG.uniform(-3, 3))
        q, d = oracle.quantize_q8_0(x)
        s = (np.abs(RNG.standard_normal(K // group)) * 0.02).astype(np.float32)
        got = float(oracle.qdot_grouped(row, bits, s, group, q, d))
        exact = oracle.qdot_grouped_f64(row, bits, s, group, q, d)
        parts = np.array([oracle.block_partial(row, bits, q, b) for b in range(K // 32)], np.float64)
        coef = np.repeat(s.astype(np.float64), group // 32) * d.astype(np.float64)
        n = K // 32 + 2
        bound = (n * U / (1 - n * U)) * float(np.sum(np.abs(coef * parts)))
        assert abs(got - exact) <= bound + 1e-30, (trial, got, exact, bound)


# ---------------------------------------------------------------------------
# exp and SiLU
# ---------------------------------------------------------------------------

def test_cexp_within_two_ulp_of_exp():
    z = np.concatenate([RNG.uniform(-87.0, 88.0, 400000), np.linspace(-87, 88, 100001),
                        RNG.uniform(-1, 1, 100000)]).astype(np.float32)
    got = oracle.cexp(z).astype(np.float64)
    ref = np.exp(z.astype(np.float64))
    ulps = np.abs(got - ref) / np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert ulps.max() <= 2.0, float(ulps.max())


def test_cexp_special_values():
    out = oracle.cexp(np.array([0.0, 88.5, 100.0, -87.5, -200.0, math.log(2) * 10], np.float32))
    assert out[0] == 1.0
    assert math.isinf(out[1]) and math.isinf(out[2])
    assert out[3] == 0.0 and out[4] == 0.0
    assert abs(out[5] - 1024.0) <= 2 * ulp32(1024.0)


def test_silu_special_cases_and_accuracy():
    g = np.array([0.0, 20.0, 31.75, 1000.0, -88.5, -127.0], np.float32)
    s = oracle.silu(g)
    assert s[0] == 0.0
    assert s[1] == 20.0 and s[2] == 31.75 and s[3] == 1000.0
    assert s[4] == 0.0 and math.copysign(1.0, s[4]) < 0  # -0
    assert s[5] == 0.0 and math.copysign(1.0, s[5]) < 0
    gg = RNG.uniform(-80, 80, 200000).astype(np.float32)
    got = oracle.silu(gg).astype(np.float64)
    g64 = gg.astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64))
    tiny = np.abs(ref) < 1e-30
    ulps = np.abs(got - ref)[~tiny] / np.spacing(ref[~tiny].astype(np.float32)).astype(np.float64)
    assert ulps.max() <= 4.0


# ---------------------------------------------------------------------------
# Router (README sigmoid-router item)
# ---------------------------------------------------------------------------

def _router_case(E=16, H=64, scale=1.0):
    W = (RNG.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    x = (RNG.standard_normal(H) * scale).astype(np.float32)
    b = (RNG.standard_normal(E) * 0.3).astype(np.float32)
    return x, W, b


def test_router_scores_and_brute_force_selection():
    for trial in range(50):
        x, W, b = _router_case()
        k = int(RNG.integers(1, 9))
        r = oracle.route_token(x, W, b, k, 2.5)
        logit = W.astype(np.float64) @ x.astype(np.float64)
        sig = 1.0 / (1.0 + np.exp(-logit))
        assert np.all(np.abs(r["s"] - sig) <= 4 * np.spacing(sig.astype(np.float32)))
        assert np.array_equal(r["c"], (r["s"] + b).astype(np.float32))
        c = r["c"]
        chosen = set()
        for e in range(16):
            before = sum(1 for f in range(16) if c[f] > c[e] or (c[f] == c[e] and f < e))
            if before < k:
                chosen.add(e)
        assert set(r["ids"].tolist()) == chosen
        # slot order = selection order (score descending, lower id first)
        order = sorted(chosen, key=lambda e: (-float(c[e]), e))
        assert r["ids"].tolist() == order
        # weights: renormalised unbiased scores times rsf
        assert abs(r["w"].sum() - 2.5) <= 4 * k * 2.5 * 2.0 ** -52
        s_sel = r["s"][r["ids"]].astype(np.float64)
        assert np.allclose(r["w"], 2.5 * s_sel / s_sel.sum(), rtol=1e-15)
        rest = [float(c[e]) for e in range(16) if e not in chosen]
        assert r["gap"] == np.float32(float(c[order[-1]]) - max(rest))


def test_router_bias_selects_but_does_not_weight():
    x, W, b = _router_case()
    b = np.zeros(16, np.float32)
    b[5], b[11] = 10.0, 9.0  # force experts 5 and 11 to the top
    r = oracle.route_token(x, W, b, 2, 1.0)
    assert r["ids"].tolist() == [5, 11]
    s = r["s"].astype(np.float64)
    assert np.allclose(r["w"], [s[5] / (s[5] + s[11]), s[11] / (s[5] + s[11])], rtol=1e-15)


def test_router_ties_go_to_lower_id():
    W = np.tile(RNG.standard_normal((1, 64)).astype(np.float32), (8, 1))
    x = RNG.standard_normal(64).astype(np.float32)
    r = oracle.route_token(x, W, np.zeros(8, np.float32), 3, 1.0)
    assert r["ids"].tolist() == [0, 1, 2]
    assert np.allclose(r["w"], [1 / 3] * 3, rtol=1e-15)


def test_router_k_equals_E_is_full_normalisation():
    x, W, _ = _router_case(E=8)
    r = oracle.route_token(x, W, np.zeros(8, np.float32), 8, 2.5)
    s = r["s"].astype(np.float64)
    assert sorted(r["ids"].tolist()) == list(range(8))
    for j, e in enumerate(r["ids"]):
        assert abs(r["w"][j] - 2.5 * s[e] / s.sum()) <= 1e-15
    assert math.isinf(r["gap"])


# ---------------------------------------------------------------------------
# Router variants: group-limited selection and adaptive expert top-p
# ---------------------------------------------------------------------------

def _flat_router(bias):
    """W = 0: every logit is 0 and every s is exactly 1/2, so c = 1/2 + bias."""
    E = bias.shape[0]
    return np.zeros(8, np.float32), np.zeros((E, 8), np.float32), bias.astype(np.float32)


def test_router_group_stage_off_is_plain_top_k():
    for trial in range(20):
        x, W, b = _router_case(E=32)
        k = int(RNG.integers(1, 9))
        plain = oracle.route_token(x, W, b, k, 2.5)
        for opts in (oracle.route_opts(1, 1, 1.0), oracle.route_opts(4, 4, 1.0), oracle.route_opts(8, 8, 1.0)):
            r = oracle.route_token(x, W, b, k, 2.5, opts)
            assert np.array_equal(r["ids"], plain["ids"])
            assert np.array_equal(r["w"], plain["w"])


def test_router_group_stage_hand_example():
    # groups {0,1} {2,3} {4,5} {6,7}; c = 0.5 + bias
    b = np.array([0.9, -0.4, 0.5, 0.45, 0.4, 0.4, -0.1, 0.0])
    x, W, b = _flat_router(b)
    # group scores (top-2 sums): 1.5, 1.95, 1.8, 0.9 -> groups 1 and 2 kept;
    # expert 0 has the best single score but its group is dropped
    r = oracle.route_token(x, W, b, 2, 2.0, oracle.route_opts(4, 2, 1.0))
    assert r["ids"].tolist() == [2, 3]
    assert r["w"].tolist() == [1.0, 1.0]
    plain = oracle.route_token(x, W, b, 2, 2.0)
    assert plain["ids"].tolist() == [0, 2]
    # a tie between group scores keeps the lower group
    b2 = np.array([0.3, 0.2, 0.0, 0.0, 0.3, 0.2, 0.0, 0.0])
    x, W, b2 = _flat_router(b2)
    r = oracle.route_token(x, W, b2, 2, 1.0, oracle.route_opts(4, 1, 1.0))
    assert r["ids"].tolist() == [0, 1]


def test_router_group_stage_invariants():
    for trial in range(60):
        E = 32
        n_group = int(RNG.choice([2, 4, 8]))
        gsz = E // n_group
        topk_group = int(RNG.integers(1, n_group + 1))
        k = int(RNG.integers(1, min(8, topk_group * gsz) + 1))
        x, W, b = _router_case(E=E)
        r = oracle.route_token(x, W, b, k, 2.5, oracle.route_opts(n_group, topk_group, 1.0))
        c = r["c"]
        # group scores from a sort (independent of the oracle's running top-2)
        score = np.array([np.float32(np.sort(c[g * gsz:(g + 1) * gsz])[-1]) +
                          np.float32(np.sort(c[g * gsz:(g + 1) * gsz])[-2]) for g in range(n_group)], np.float32)
        kept = sorted(range(n_group), key=lambda g: (-float(score[g]), g))[:topk_group]
        eligible = [e for e in range(E) if e // gsz in kept]
        assert all(int(e) // gsz in kept for e in r["ids"])
        # brute force over the eligible experts: e is chosen iff fewer than k precede it
        chosen = [e for e in eligible
                  if sum(1 for f in eligible if c[f] > c[e] or (c[f] == c[e] and f < e)) < k]
        assert r["ids"].tolist() == sorted(chosen, key=lambda e: (-float(c[e]), e))
        assert abs(r["w"].sum() - 2.5) <= 1e-12
        assert r["gap"] > 0


def test_router_top_p_limits():
    for trial in range(20):
        x, W, b = _router_case(E=32)
        k = int(RNG.integers(2, 9))
        plain = oracle.route_token(x, W, b, k, 2.5)
        full = oracle.route_token(x, W, b, k, 2.5, oracle.route_opts(1, 1, 1.0))
        assert np.array_equal(full["ids"], plain["ids"]) and np.array_equal(full["w"], plain["w"])
        one = oracle.route_token(x, W, b, k, 2.5, oracle.route_opts(1, 1, 1e-6))
        s = plain["s"][plain["ids"]]
        top = int(np.argmax(s))  # first slot with the largest s
        assert [j for j in range(k) if one["ids"][j] >= 0] == [top]
        assert one["ids"][top] == plain["ids"][top] and one["w"][top] == 2.5
        assert all(one["w"][j] == 0.0 for j in range(k) if j != top)


def test_router_top_p_invariants():
    for trial in range(80):
        x, W, b = _router_case(E=32)
        k = int(RNG.integers(2, 9))
        p = float(RNG.uniform(0.05, 0.99))
        plain = oracle.route_token(x, W, b, k, 2.5)
        r = oracle.route_token(x, W, b, k, 2.5, oracle.route_opts(1, 1, p))
        s = plain["s"][plain["ids"]].astype(np.float64)
        kept = [j for j in range(k) if r["ids"][j] >= 0]
        dropped = [j for j in range(k) if r["ids"][j] < 0]
        assert kept  # at least one slot
        # kept slots keep their experts and positions; they hold the largest s
        assert all(r["ids"][j] == plain["ids"][j] for j in kept)
        if dropped:
            assert min(s[kept]) >= max(s[dropped])
        # weights renormalised over the kept slots
        assert abs(r["w"].sum() - 2.5) <= 1e-12
        assert all(r["w"][j] == 0.0 for j in dropped)
        assert np.allclose(r["w"][kept], 2.5 * s[kept] / s[kept].sum(), rtol=1e-15)
        # the cut is the shortest prefix reaching p (fp64 shares, fp32 slack)
        share = np.sort(s)[::-1] / s.sum()
        m = len(kept)
        assert share[:m].sum() >= p - 1e-6
        if m > 1:
            assert share[:m - 1].sum() < p + 1e-6


def test_router_top_p_monotone_in_p():
    x, W, b = _router_case(E=32)
    counts = []
    for p in np.linspace(0.01, 0.99, 40):
        r = oracle.route_token(x, W, b, 8, 1.0, oracle.route_opts(1, 1, float(p)))
        counts.append(int(np.sum(r["ids"] >= 0)))
    assert counts == sorted(counts) and counts[0] == 1


def test_dispatch_skips_dropped_slots():
    for trial in range(20):
        S, k, E = int(RNG.integers(1, 30)), int(RNG.integers(2, 5)), int(RNG.integers(4, 20))
        ids = np.stack([RNG.choice(E, size=k, replace=False) for _ in range(S)]).astype(np.int32)
        drop = RNG.random(ids.shape) < 0.3
        ids[drop] = -1
        r = oracle.dispatch(ids, E)
        flat = ids.reshape(-1)
        valid = [p for p in range(S * k) if flat[p] >= 0]
        assert r["offsets"][E] == len(valid)
        assert sorted(r["sorted"][:len(valid)].tolist()) == valid
        for p in range(S * k):
            if flat[p] < 0:
                assert r["inv"][p] == -1
            else:
                assert r["sorted"][r["inv"][p]] == p


# ---------------------------------------------------------------------------
# Union dispatch (README batched-union item)
# ---------------------------------------------------------------------------

def test_dispatch_brute_force():
    for trial in range(30):
        S, k, E = int(RNG.integers(1, 40)), int(RNG.integers(1, 5)), int(RNG.integers(4, 20))
        ids = np.stack([RNG.choice(E, size=k, replace=False) for _ in range(S)]).astype(np.int32)
        r = oracle.dispatch(ids, E)
        flat = ids.reshape(-1)
        P = S * k
        for e in range(E + 1):
            assert r["offsets"][e] == int(np.sum(flat < e))
        assert r["offsets"][E] == P
        for e in range(E):
            members = [p for p in range(P) if flat[p] == e]  # ascending p
            got = r["sorted"][r["offsets"][e]:r["offsets"][e + 1]].tolist()
            assert got == members
        assert sorted(r["sorted"].tolist()) == list(range(P))
        for p in range(P):
            assert r["sorted"][r["inv"][p]] == p
        assert r["active"].tolist() == sorted(set(flat.tolist()))
        assert r["n_active"] == len(set(flat.tolist()))


# ---------------------------------------------------------------------------
# One expert on one token
# ---------------------------------------------------------------------------

def _tiny_bank(bits, n_mat, rows, K, lo, hi):
    data, scale = [], []
    for m in range(n_mat):
        codes = RNG.integers(lo, hi + 1, size=(rows, K)).astype(np.int8)
        data.append(np.stack([oracle.pack_row(r, bits) for r in codes]))
        scale.append((np.abs(RNG.standard_normal(rows)) * 0.02).astype(np.float32))
    return synth.Bank(n_mat, rows, K, bits, data, scale), data, scale


def _repack(bank_, bits_from, bits_to):
    data = [np.stack([oracle.pack_row(oracle.unpack_row(r, bits_from, bank_.K), bits_to)
                      for r in m]) for m in bank_.data]
    return synth.Bank(bank_.n_mat, bank_.rows, bank_.K, bits_to, data, bank_.scale)


@pytest.mark.parametrize("bits,lo,hi", [(4, -8, 7), (2, -2, 1)])
def test_expert_packed_equals_int8_container(bits, lo, hi):
    H, I = 128, 96
    g, _, _ = _tiny_bank(bits, 2, I, H, lo, hi)
    u, _, _ = _tiny_bank(bits, 2, I, H, lo, hi)
    d, _, _ = _tiny_bank(bits, 2, H, I, lo, hi)
    x = RNG.standard_normal(H).astype(np.float32)
    xq, xd = oracle.quantize_q8_0(x)
    a = oracle.expert_ffn(g, u, d, 1, xq, xd)
    b = oracle.expert_ffn(_repack(g, bits, 8), _repack(u, bits, 8), _repack(d, bits, 8), 1, xq, xd)
    for key in ("g", "u", "h", "hq", "hd", "y"):
        assert a[key].tobytes() == b[key].tobytes(), key


def test_expert_against_fp64_shadow():
    H, I = 256, 128
    g, _, _ = _tiny_bank(8, 1, I, H, -127, 127)
    u, _, _ = _tiny_bank(8, 1, I, H, -127, 127)
    d, _, _ = _tiny_bank(8, 1, H, I, -127, 127)
    x = RNG.standard_normal(H).astype(np.float32)
    xq, xd = oracle.quantize_q8_0(x)
    r = oracle.expert_ffn(g, u, d, 0, xq, xd)

    def bound(row, scale, q, dd):
        K = q.size
        parts = np.array([oracle.block_partial(row, 8, q, b) for b in range(K // 32)], np.float64)
        n = K // 32 + 1
        return (n * U / (1 - n * U)) * scale * float(np.sum(np.abs(dd.astype(np.float64) * parts)))

    for i in range(I):
        for bank_, key in ((g, "g"), (u, "u")):
            row, sc = bank_.data[0][i], float(bank_.scale[0][i])
            v64 = oracle.qdot_f64(row, 8, sc, xq, xd)
            assert abs(r[key][i] - v64) <= bound(row, sc, xq, xd) + 1e-30
        h64 = float(r["g"][i]) / (1.0 + math.exp(-float(r["g"][i]))) * float(r["u"][i])
        assert abs(r["h"][i] - h64) <= 4 * ulp32(h64) + 1e-30
    hq, hd = oracle.quantize_q8_0(r["h"])
    assert np.array_equal(hq, r["hq"]) and np.array_equal(hd, r["hd"])
    for n in range(H):
        row, sc = d.data[0][n], float(d.scale[0][n])
        y64 = oracle.qdot_f64(row, 8, sc, r["hq"], r["hd"])
        assert abs(r["y"][n] - y64) <= bound(row, sc, r["hq"], r["hd"]) + 1e-30


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [8, 4, 2])
def test_hand_two_expert_example(bits):
    fx = hand_example.load()
    L = hand_example.layer(bits=bits)
    x = hand_example.x_values()[None, :]
    r = oracle.layer_forward(L, x)
    assert r["ids"][0].tolist() == [0, 1]
    assert r["w"][0].tolist() == [1.25, 1.25]
    assert np.all(r["xd"] == 1.0) and np.array_equal(r["xq"][0].astype(np.float32), x[0])
    y0, y1 = hand_example.y_closed(0), hand_example.y_closed(1)
    out = hand_example.out_closed()
    for n in range(64):
        assert Fraction(float(r["y_routed"][0, n])) == y0[n]
        assert Fraction(float(r["y_routed"][1, n])) == y1[n]
        assert Fraction(float(r["out"][0, n])) == out[n]
    hv = fx["hand_values"]
    for n, v in hv["out"].items():
        assert r["out"][0, int(n)] == v
    for n, v in hv["y0"].items():
        assert r["y_routed"][0, int(n)] == v
    for n, v in hv["y1"].items():
        assert r["y_routed"][1, int(n)] == v
    # per-expert intermediate codes match the closed form
    xq, xd = oracle.quantize_q8_0(x[0])
    for e in range(2):
        f = oracle.expert_ffn(L.gate, L.up, L.down, e, xq, xd)
        assert f["hq"].tolist() == hand_example.hq_closed(e)
        assert np.all(f["hd"] == np.float32(127.0 / 32.0))


def test_hand_example_bias_flips_slot_order_not_weights():
    L = hand_example.layer(bits=4, bias=(0.0, 0.5))
    r = oracle.layer_forward(L, hand_example.x_values()[None, :])
    assert r["ids"][0].tolist() == [1, 0]
    assert r["w"][0].tolist() == [1.25, 1.25]
    out = hand_example.out_closed()
    assert all(Fraction(float(r["out"][0, n])) == out[n] for n in range(64))


def test_hand_example_with_shared_expert():
    L = hand_example.layer(bits=8, with_shared=True)
    r = oracle.layer_forward(L, hand_example.x_values()[None, :])
    out = hand_example.out_closed(with_shared=True)
    assert all(Fraction(float(r["out"][0, n])) == out[n] for n in range(64))


def _q8_0_f64(v):
    """Q8_0 of a vector evaluated in fp64 with a division (a different
    formulation from the oracle's fp32 multiply by the reciprocal)."""
    v = v.reshape(-1, 32)
    amax = np.max(np.abs(v), axis=1, keepdims=True)
    dd = amax / 127.0
    t = np.divide(v, dd, out=np.zeros_like(v), where=dd > 0)
    q = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127)
    return (q * dd).reshape(-1)


def _naive_dense_layer(L, x):
    """Deliberately naive fp64 formulation: dense loop over every expert with a
    0/1 selection mask, weights dequantised to fp64, unblocked dot products,
    the intermediate requantised in fp64.  It checks structure (which experts,
    which weights, shared term, scaling); rounding differences can only flip
    an intermediate code now and then (a few 1e-3 of the output RMS each)."""
    w = L.w
    E, H, I, k = w.n_experts, w.hidden, w.inter, w.top_k
    W = L.router_w.numpy().astype(np.float64)
    bias = L.bias.numpy().astype(np.float64)

    def deq(bank_, m):
        rows = np.stack([oracle.unpack_row(r, bank_.bits, bank_.K) for r in np.asarray(bank_.data[m])])
        sc = np.asarray(bank_.scale[m], np.float64)
        if bank_.group:  # weight of column c = scale of its group * code
            return rows.astype(np.float64) * np.repeat(sc.reshape(bank_.rows, -1), bank_.group, axis=1)
        return rows.astype(np.float64) * sc[:, None]

    mats = [(deq(L.gate, e), deq(L.up, e), deq(L.down, e)) for e in range(E)]
    sh = (deq(L.sh_gate, 0), deq(L.sh_up, 0), deq(L.sh_down, 0)) if w.has_shared else None
    out = np.zeros((x.shape[0], H))
    for t in range(x.shape[0]):
        xq, xd = oracle.quantize_q8_0(x[t])
        xt = xq.astype(np.float64) * np.repeat(xd.astype(np.float64), 32)
        s = 1.0 / (1.0 + np.exp(-(W @ x[t].astype(np.float64))))
        c = s + bias
        order = sorted(range(E), key=lambda e: (-c[e], e))
        mask = np.zeros(E)
        mask[order[:k]] = 1.0
        denom = float(np.sum(mask * s))
        for e in range(E):
            g, u, d = mats[e]
            gg, uu = g @ xt, u @ xt
            h = _q8_0_f64(gg / (1.0 + np.exp(-gg)) * uu)
            out[t] += mask[e] * w.rsf * s[e] / denom * (d @ h)
        if sh is not None:
            g, u, d = sh
            gg, uu = g @ xt, u @ xt
            out[t] += d @ _q8_0_f64(gg / (1.0 + np.exp(-gg)) * uu)
    return out


@pytest.mark.parametrize("variant", ["tiny", "tiny_shared_rsf", "tiny_int4", "tiny_int2", "tiny_group32",
                                     "tiny_int4_group128", "tiny_int2_group64"])
def test_layer_against_naive_dense_path(variant):
    base = synth.WORKLOADS["tiny"]
    w = {"tiny": base,
         "tiny_shared_rsf": synth.scaled(base, name="tiny_sh", has_shared=True, rsf=2.5, top_k=3),
         "tiny_int4": synth.scaled(base, name="tiny4", layer="tiny_int4", bits=4, rsf=2.5),
         "tiny_int2": synth.scaled(base, name="tiny2", layer="tiny_int2", bits=2, has_shared=True),
         "tiny_group32": synth.scaled(base, name="tiny_g32", layer="tiny_g32", group=32, has_shared=True),
         "tiny_int4_group128": synth.scaled(base, name="tiny4_g128", layer="tiny4_g128", bits=4, group=128,
                                            rsf=2.5),
         "tiny_int2_group64": synth.scaled(base, name="tiny2_g64", layer="tiny2_g64", bits=2, group=64,
                                           has_shared=True)}[variant]
    L = synth.make_layer(w)
    x = synth.activations(w).numpy()
    r = oracle.layer_forward(L, x)
    naive = _naive_dense_layer(L, x)
    rms = math.sqrt(float(np.mean(naive ** 2)))
    diff = np.abs(r["out"] - naive)
    assert np.max(diff) <= 1e-2 * rms
    assert math.sqrt(float(np.mean(diff ** 2))) <= 1e-3 * rms


def test_layer_rsf_zero_gives_shared_only():
    w = synth.scaled(synth.WORKLOADS["tiny"], name="tiny_rsf0", has_shared=True, rsf=0.0)
    L = synth.make_layer(w)
    x = synth.activations(w).numpy()
    r = oracle.layer_forward(L, x)
    assert np.array_equal(r["out"], r["y_shared"].astype(np.float64))


def test_layer_single_expert_no_shared():
    w = synth.scaled(synth.WORKLOADS["tiny"], name="tiny_k1", top_k=1, rsf=1.75)
    L = synth.make_layer(w)
    x = synth.activations(w).numpy()
    r = oracle.layer_forward(L, x)
    assert np.all(r["w"] == 1.75)
    assert np.array_equal(r["out"], 1.75 * r["y_routed"].astype(np.float64))


def test_layer_traces_agree_with_expert_function():
    w = synth.WORKLOADS["tiny"]
    L = synth.make_layer(w)
    x = synth.activations(w).numpy()
    r = oracle.layer_forward(L, x)
    for t in range(w.S):
        for j in range(w.top_k):
            f = oracle.expert_ffn(L.gate, L.up, L.down, int(r["ids"][t, j]), r["xq"][t], r["xd"][t])
            assert f["y"].tobytes() == r["y_routed"][t * w.top_k + j].tobytes()


@pytest.mark.parametrize("n_group,topk_group,top_p", [(4, 2, 1.0), (1, 1, 0.6), (4, 3, 0.5)])
def test_layer_with_router_variants_composes(n_group, topk_group, top_p):
    """The layer with group-limited selection / top-p equals the shared output
    plus the router's kept slots weighted over the expert function (fp64)."""
    w = synth.scaled(synth.WORKLOADS["tiny"], name="tiny_rv", has_shared=True, rsf=2.5, top_k=4,
                     n_group=n_group, topk_group=topk_group, top_p=top_p)
    L = synth.make_layer(w)
    x = synth.activations(w).numpy()
    r = oracle.layer_forward(L, x)
    opts = oracle.route_opts(n_group, topk_group, top_p)
    G, U, D = oracle.bank(L.gate), oracle.bank(L.up), oracle.bank(L.down)
    SG, SU, SD = oracle.bank(L.sh_gate), oracle.bank(L.sh_up), oracle.bank(L.sh_down)
    n_dropped = 0
    for t in range(w.S):
        rt = oracle.route_token(x[t], L.router_w, L.bias, w.top_k, w.rsf, opts)
        assert np.array_equal(rt["ids"], r["ids"][t])
        q, dq = oracle.quantize_q8_0(x[t][None, :])
        want = oracle.expert_ffn(SG, SU, SD, 0, q[0], dq[0])["y"].astype(np.float64)
        for j in range(w.top_k):
            if rt["ids"][j] < 0:
                n_dropped += 1
                continue
            y = oracle.expert_ffn(G, U, D, int(rt["ids"][j]), q[0], dq[0])["y"].astype(np.float64)
            want = want + rt["w"][j] * y
        assert np.array_equal(r["out"][t], want)
    if top_p < 1.0:
        assert n_dropped > 0


# ---------------------------------------------------------------------------
# The input generator
# ---------------------------------------------------------------------------

def test_splitmix64_matches_published_sequence():
    # Reference sequence of SplitMix64 seeded with 1234567 (state advanced by
    # the golden gamma before each output).
    state = 1234567
    gamma = 0x9E3779B97F4A7C15
    words = [synth.mix64_int((state + (i + 1) * gamma) & ((1 << 64) - 1)) for i in range(3)]
    assert words[0] == 6457827717110365317
    assert words[1] == 3203168211198807973
    t = synth.random_u64(1234567, 3).numpy().view(np.uint64).tolist()
    assert t == words


def test_generator_deterministic_and_streams_independent():
    a = synth.random_bytes(synth.stream_key("a"), 1000)
    b = synth.random_bytes(synth.stream_key("a"), 1000)
    c = synth.random_bytes(synth.stream_key("b"), 1000)
    assert torch.equal(a, b) and not torch.equal(a, c)
    codes = synth.random_int8_codes(synth.stream_key("c"), 200000)
    assert int(codes.min()) == -127 and int(codes.max()) == 127
    z = synth.normal(synth.stream_key("n"), 100000)
    assert abs(float(z.mean())) < 0.02 and abs(float(z.std()) - 1.0) < 0.02

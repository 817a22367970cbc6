"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: libm in
float64, exact error bounds, closed forms, brute force, the pages' worked
examples (tests/golden/), numpy float64 matmuls, and invariants.  No GPU.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def ulp32(x):
    """Spacing of float32 at |x| (subnormal spacing below 2^-126)."""
    x = abs(x)
    if x < 2.0 ** -126:
        return 2.0 ** -149
    return 2.0 ** (math.floor(math.log2(x)) - 23)


# --------------------------------------------------------------------------
# exp_spec and sigmoid_spec: error bound against libm float64.
# --------------------------------------------------------------------------

def _sweep():
    ys = np.linspace(-30.0, 30.0, 60001, dtype=np.float64)
    rng = np.random.default_rng(7)
    extra = rng.uniform(-104.0, 89.0, 20000)
    return np.concatenate([ys, extra]).astype(np.float32)


def test_exp_spec_within_2ulp_of_libm():
    worst = 0.0
    for y in _sweep():
        y = float(y)
        got = oracle.exp_spec(y)
        ref = math.exp(y) if y < 88.7 else None
        if ref is None or ref > 3.4028234663852886e38:
            continue
        err = abs(got - ref) / ulp32(ref)
        worst = max(worst, err)
    assert worst <= 2.0, worst


def test_exp_spec_special_values():
    assert oracle.exp_spec(0.0) == 1.0
    assert oracle.exp_spec(-0.0) == 1.0
    assert oracle.exp_spec(1.0) == f32(math.e)
    assert math.isinf(oracle.exp_spec(89.5))
    assert oracle.exp_spec(-105.0) == 0.0
    # near the top of the range the value is finite and within 2 ulp
    for y in (88.0, 88.5, 88.72):
        ref = math.exp(f32(y))
        assert abs(oracle.exp_spec(y) - ref) <= 2 * ulp32(ref)
    # subnormal results: within 1 subnormal spacing
    for y in (-88.0, -95.0, -100.0, -103.0):
        ref = math.exp(f32(y))
        assert abs(oracle.exp_spec(y) - ref) <= 2.0 ** -149


def test_exp_spec_monotone():
    ys = np.sort(_sweep())
    vals = [oracle.exp_spec(float(y)) for y in ys]
    assert all(b >= a for a, b in zip(vals, vals[1:]))


def test_sigmoid_spec_within_3ulp_and_symmetric():
    worst = 0.0
    for z in np.linspace(-40.0, 40.0, 40001, dtype=np.float32):
        z = float(z)
        ref = 1.0 / (1.0 + math.exp(-z))
        got = oracle.sigmoid_spec(z)
        worst = max(worst, abs(got - ref) / ulp32(ref))
    assert worst <= 3.0, worst
    assert oracle.sigmoid_spec(0.0) == 0.5
    assert oracle.sigmoid_spec(100.0) == 1.0
    assert oracle.sigmoid_spec(-200.0) == 0.0
    for z in (0.25, 1.0, 3.0, 7.5):
        assert abs(oracle.sigmoid_spec(z) + oracle.sigmoid_spec(-z) - 1.0) <= 2 ** -23


def test_sigmoid_spec_monotone():
    zs = np.linspace(-20, 20, 20001, dtype=np.float32)
    vals = [oracle.sigmoid_spec(float(z)) for z in zs]
    assert all(b >= a for a, b in zip(vals, vals[1:]))


# --------------------------------------------------------------------------
# Router logits: error bound against float64, closed forms.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("h,E,T", [(64, 8, 4), (2048, 64, 3), (6144, 16, 2)])
def test_router_logits_error_bound(h, E, T):
    rng = np.random.default_rng(h + E)
    x = rng.standard_normal((T, h)).astype(np.float32)
    wr = (0.02 * rng.standard_normal((h, E))).astype(np.float32)
    got = oracle.router_logits(x, wr).astype(np.float64)
    ref = x.astype(np.float64) @ wr.astype(np.float64)
    mag = np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64))
    # each lane chain has h/64 fma roundings, then 6 butterfly additions
    gamma = (h // 64 + 6) * 2.0 ** -24
    assert np.all(np.abs(got - ref) <= gamma * mag * 1.0001)


def test_router_logits_closed_forms():
    h, E = 128, 8
    rng = np.random.default_rng(3)
    wr = rng.standard_normal((h, E)).astype(np.float32)
    # unit vectors select rows of the router exactly
    for i in (0, 1, 63, 64, 127):
        x = np.zeros((1, h), np.float32)
        x[0, i] = 1.0
        assert np.array_equal(oracle.router_logits(x, wr)[0], wr[i])
    # small integers: every partial sum is exact
    xi = rng.integers(-4, 5, (3, h)).astype(np.float32)
    wi = rng.integers(-4, 5, (h, E)).astype(np.float32)
    assert np.array_equal(oracle.router_logits(xi, wi), (xi.astype(np.int64) @ wi.astype(np.int64)).astype(np.float32))


# --------------------------------------------------------------------------
# Selection: brute force full sort, ties, weight invariants.
# --------------------------------------------------------------------------

def _brute_select(logits, bias, k, rsf):
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    for t in range(T):
        s = [np.float32(oracle.sigmoid_spec(float(v))) for v in logits[t]]
        c = [np.float32(s[e] + (np.float32(0) if bias is None else bias[e])) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-float(c[e]), e))[:k]
        idx[t] = order
        den = np.float32(0)
        for e in order:
            den = np.float32(den + s[e])
        w[t] = [np.float32(np.float32(s[e] / den) * np.float32(rsf)) for e in order]
    return idx, w


@pytest.mark.parametrize("E,k,rsf", [(8, 2, 1.0), (64, 8, 1.0), (256, 8, 2.5), (16, 16, 1.5), (5, 1, 1.0)])
def test_select_matches_brute_force(E, k, rsf):
    rng = np.random.default_rng(E * 31 + k)
    T = 24
    logits = (1.6 * rng.standard_normal((T, E))).astype(np.float32)
    bias = (0.05 * rng.standard_normal(E)).astype(np.float32)
    idx, w = oracle.select(logits, bias, k, rsf)
    bi, bw = _brute_select(logits, bias, k, rsf)
    assert np.array_equal(idx, bi)
    assert np.array_equal(w.view(np.uint32), bw.view(np.uint32))


def test_select_tie_break_by_lowest_index():
    E, k = 16, 4
    logits = np.zeros((3, E), np.float32)
    bias = np.zeros(E, np.float32)
    # token 0: all keys equal -> experts 0..3
    # token 1: experts 9, 4, 12 share the largest key -> 4, 9, 12, then 0
    logits[1, [4, 9, 12]] = 2.0
    # token 2: equal sigmoid but a bias lifts 15 above the rest
    bias2 = bias.copy()
    idx, _ = oracle.select(logits, bias, k, 1.0)
    assert idx[0].tolist() == [0, 1, 2, 3]
    assert idx[1].tolist() == [4, 9, 12, 0]
    bias2[15] = 0.25
    idx2, _ = oracle.select(logits[2:3], bias2, k, 1.0)
    assert idx2[0].tolist() == [15, 0, 1, 2]


def test_select_bias_only_selects():
    """The bias changes which experts win, not the weights: with a large bias
    on expert 7 it is selected and its weight uses its unbiased score."""
    E, k = 8, 2
    logits = np.array([[3.0, 2.0, 1.0, 0.0, -1.0, -2.0, -3.0, -4.0]], np.float32)
    bias = np.zeros(E, np.float32)
    bias[7] = 10.0
    idx, w = oracle.select(logits, bias, k, 1.0)
    assert idx[0].tolist() == [7, 0]
    s7, s0 = 1 / (1 + math.exp(4.0)), 1 / (1 + math.exp(-3.0))
    assert abs(w[0, 0] - s7 / (s7 + s0)) < 1e-6
    assert abs(w[0, 1] - s0 / (s7 + s0)) < 1e-6


def test_select_weight_invariants():
    rng = np.random.default_rng(11)
    E, k, rsf, T = 256, 8, 2.5, 64
    logits = (1.6 * rng.standard_normal((T, E))).astype(np.float32)
    bias = (0.05 * rng.standard_normal(E)).astype(np.float32)
    idx, w = oracle.select(logits, bias, k, rsf)
    assert np.all(w > 0)
    sums = w.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(sums - rsf) <= 2 * k * 2.0 ** -23 * rsf)
    s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    for t in range(T):
        st = s[t, idx[t]]
        ratio = (w[t] / w[t, 0]).astype(np.float64)
        assert np.allclose(ratio, st / st[0], rtol=2e-6, atol=0)


def test_select_equal_scores_split_evenly():
    """Closed form: k equal scores give weight rsf / k each."""
    logits = np.zeros((1, 8), np.float32)
    _, w = oracle.select(logits, None, 2, 1.0)
    assert w[0].tolist() == [0.5, 0.5]
    _, w = oracle.select(logits, None, 4, 2.0)
    assert w[0].tolist() == [0.5, 0.5, 0.5, 0.5]


def test_n_group_one_equals_plain_topk():
    """n_group = 1: one group holding every expert; the group-limited stage
    keeps it, so selection is the plain top-k over all experts -- which is
    what the brute force above computes.  Here: the winners are exactly the
    k largest keys of the whole row."""
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((10, 32)).astype(np.float32)
    idx, _ = oracle.select(logits, None, 6, 1.0)
    for t in range(10):
        assert set(idx[t]) == set(np.argsort(-logits[t], kind="stable")[:6])


# --------------------------------------------------------------------------
# Run-time routing limits: explicit smaller k, adaptive expert top-p.
# --------------------------------------------------------------------------

def test_limits_off_equal_plain_selection():
    rng = np.random.default_rng(41)
    logits = (1.6 * rng.standard_normal((20, 64))).astype(np.float32)
    bias = (0.05 * rng.standard_normal(64)).astype(np.float32)
    i0, w0 = oracle.select(logits, bias, 8, 2.5)
    i1, w1 = oracle.select(logits, bias, 8, 2.5, k_use=8, top_p=1.0)
    assert np.array_equal(i0, i1) and np.array_equal(w0.view(np.uint32), w1.view(np.uint32))


@pytest.mark.parametrize("E,k,k_use", [(64, 8, 4), (256, 8, 1), (16, 6, 5)])
def test_smaller_k_is_brute_force_topk_of_that_k(E, k, k_use):
    """An explicit smaller k routes exactly like a layer built with that k
    (brute-force full sort), in the first k_use slots; the rest are dropped."""
    rng = np.random.default_rng(E + k_use)
    T = 12
    logits = (1.6 * rng.standard_normal((T, E))).astype(np.float32)
    bias = (0.05 * rng.standard_normal(E)).astype(np.float32)
    idx, w = oracle.select(logits, bias, k, 1.5, k_use=k_use)
    bi, bw = _brute_select(logits, bias, k_use, 1.5)
    assert np.array_equal(idx[:, :k_use], bi)
    assert np.array_equal(w[:, :k_use].view(np.uint32), bw.view(np.uint32))
    assert np.all(idx[:, k_use:] == -1) and np.all(w[:, k_use:] == 0)


def test_top_p_closed_forms():
    """Scores that are exact in float32: a logit of 20 gives s = 1 (e^-20 is
    below half an ulp of 1), a logit of 0 gives s = 1/2.  Logits
    [20, 0, 0, 20, 0, -3], no bias, k = 4: slots hold experts 0, 3, 1, 2
    (ties by index) with scores 1, 1, 1/2, 1/2, total 3.  Keeping the
    shortest prefix whose score reaches p of the total, renormalised:
      p = 0.25 -> 1 slot (1 >= 0.75), weight rsf;
      p = 0.5  -> 2 slots (2 >= 1.5), weights rsf/2 each;
      p = 2/3  -> 2 slots: float32(2/3) * 3 rounds to exactly 2, which the
                  first two slots reach (reaching the share is enough);
      p = 0.7  -> 3 slots (2 < 2.1 <= 2.5), weights 2/5, 2/5, 1/5 of rsf;
      p = 0.9  -> 4 slots (2.5 < 2.7), weights 1/3, 1/3, 1/6, 1/6 of rsf;
    and with k_use = 3 first (total 2.5), p = 0.9 -> 3 slots (2 < 2.25)."""
    logits = np.array([[20.0, 0.0, 0.0, 20.0, 0.0, -3.0]], np.float32)
    rsf = 2.5
    assert np.float32(np.float32(2 / 3) * np.float32(3)) == np.float32(2)
    cases = [(4, 0.25, [1.0]), (4, 0.5, [0.5, 0.5]), (4, 2 / 3, [0.5, 0.5]), (4, 0.7, [0.4, 0.4, 0.2]),
             (4, 0.9, [1 / 3, 1 / 3, 1 / 6, 1 / 6]), (3, 0.9, [0.4, 0.4, 0.2])]
    for k_use, p, frac in cases:
        idx, w = oracle.select(logits, None, 4, rsf, k_use=k_use, top_p=p)
        m = len(frac)
        assert idx[0].tolist() == [0, 3, 1, 2][:m] + [-1] * (4 - m), (k_use, p)
        assert np.allclose(w[0, :m], np.array(frac) * rsf, rtol=2e-7, atol=0), (k_use, p)
        assert np.all(w[0, m:] == 0)


def test_top_p_invariants_and_monotone():
    """On random scores: the kept slots are a prefix of the plain selection,
    the shortest one whose score reaches the share p (checked in float64
    with a margin of a few float32 roundings), weights sum to rsf and keep
    the ratios of the scores, and a larger p never keeps fewer slots."""
    rng = np.random.default_rng(9)
    E, k, rsf, T = 256, 8, 2.5, 48
    logits = (1.6 * rng.standard_normal((T, E))).astype(np.float32)
    bias = (0.05 * rng.standard_normal(E)).astype(np.float32)
    i_all, _ = oracle.select(logits, bias, k, rsf)
    s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    prev_m = np.ones(T, int)
    for p in (0.05, 0.3, 0.5, 0.7, 0.9, 0.99):
        idx, w = oracle.select(logits, bias, k, rsf, top_p=p)
        m = (idx >= 0).sum(axis=1)
        assert np.all(m >= 1) and np.all(m >= prev_m)
        prev_m = m
        for t in range(T):
            mt = m[t]
            assert np.array_equal(idx[t, :mt], i_all[t, :mt]) and np.all(idx[t, mt:] == -1)
            st = s[t, i_all[t]]
            cum = np.cumsum(st) / st.sum()
            margin = 1e-6
            assert cum[mt - 1] >= p - margin
            if mt > 1:
                assert cum[mt - 2] < p + margin
            assert abs(float(w[t, :mt].astype(np.float64).sum()) - rsf) <= 2 * k * 2.0 ** -23 * rsf
            assert np.allclose(w[t, :mt] / w[t, 0], st[:mt] / st[0], rtol=2e-6, atol=0)


def test_top_p_tiny_keeps_one_slot_with_weight_rsf():
    rng = np.random.default_rng(3)
    logits = (1.6 * rng.standard_normal((16, 64))).astype(np.float32)
    idx, w = oracle.select(logits, None, 8, 2.5, top_p=1e-6)
    assert np.all(idx[:, 1:] == -1) and np.all(w[:, 0] == np.float32(2.5)) and np.all(w[:, 1:] == 0)


def test_limits_reject_out_of_range():
    logits = np.zeros((2, 8), np.float32)
    for kw in (dict(k_use=0), dict(k_use=5), dict(top_p=0.0), dict(top_p=1.5), dict(top_p=-0.2)):
        with pytest.raises(ValueError, match="-2"):
            oracle.select(logits, None, 4, 1.0, **kw)


# --------------------------------------------------------------------------
# Dispatch: the pages' worked examples, invariants, brute force.
# --------------------------------------------------------------------------

def test_dispatch_worked_examples_from_pages():
    ex = json.load(open(os.path.join(GOLDEN, "dispatch_worked_examples.json")))["examples"]
    for case in ex:
        d = oracle.dispatch(np.array(case["idx"], np.int32), case["E"])
        for key in ("counts", "offsets", "sorted_ids", "inv", "active"):
            assert d[key].tolist() == case[key], (case["name"], key)
        k = case["k"]
        for e, members in case["groups"].items():
            e = int(e)
            seg = d["sorted_ids"][d["offsets"][e]:d["offsets"][e + 1]]
            assert sorted({int(a) // k for a in seg}) == sorted(members)


def _check_dispatch_invariants(idx, E, d):
    flat = idx.reshape(-1)
    n = flat.size
    off = d["offsets"]
    assert off[0] == 0 and off[E] == n and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off), d["counts"])
    assert np.array_equal(np.sort(d["sorted_ids"]), np.arange(n))
    for e in range(E):
        seg = d["sorted_ids"][off[e]:off[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    assert np.array_equal(d["sorted_ids"][d["inv"]], np.arange(n))
    assert d["active"].tolist() == [e for e in range(E) if d["counts"][e] > 0]


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (7, 2, 8), (64, 8, 256), (300, 8, 64), (33, 1, 3)])
def test_dispatch_invariants_and_brute_force(T, k, E):
    rng = np.random.default_rng(T * k + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch(idx, E)
    _check_dispatch_invariants(idx, E, d)
    flat = idx.reshape(-1)
    brute = sorted(range(flat.size), key=lambda a: flat[a])  # Python sort is stable
    assert d["sorted_ids"].tolist() == brute


def test_dispatch_skewed_and_empty():
    E = 16
    idx = np.zeros((40, 1), np.int32)  # every token to expert 0
    d = oracle.dispatch(idx, E)
    _check_dispatch_invariants(idx, E, d)
    assert d["n_active"] == 1 and d["counts"][0] == 40
    d0 = oracle.dispatch(np.zeros((0, 4), np.int32), E)
    assert d0["n_active"] == 0 and d0["offsets"].tolist() == [0] * (E + 1)


def test_dispatch_dropped_slots_follow_all_groups():
    """Dropped slots (idx -1) go to no expert: brute-force stable sort with
    the dropped key placed after every expert; offsets[E] counts the kept
    assignments and the dropped ones fill the tail in ascending order."""
    rng = np.random.default_rng(77)
    for T, k, E in ((1, 8, 256), (9, 4, 16), (64, 8, 64)):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        m = rng.integers(1, k + 1, size=T)
        for t in range(T):
            idx[t, m[t]:] = -1
        d = oracle.dispatch(idx, E)
        flat = idx.reshape(-1)
        n_kept = int((flat >= 0).sum())
        brute = sorted(range(flat.size), key=lambda a: flat[a] if flat[a] >= 0 else E)
        assert d["sorted_ids"].tolist() == brute
        off = d["offsets"]
        assert off[0] == 0 and off[E] == n_kept and np.all(np.diff(off) >= 0)
        assert np.array_equal(np.diff(off), d["counts"])
        assert d["sorted_ids"][n_kept:].tolist() == [a for a in range(flat.size) if flat[a] < 0]
        assert np.array_equal(d["sorted_ids"][d["inv"]], np.arange(flat.size))
        assert d["active"].tolist() == sorted(set(flat[flat >= 0].tolist()))
    # every slot dropped but slot 0 of one token
    idx = np.full((3, 2), -1, np.int32)
    idx[1, 0] = 5
    d = oracle.dispatch(idx, 8)
    assert d["offsets"].tolist() == [0] * 6 + [1] * 3 and d["sorted_ids"].tolist() == [2, 0, 1, 3, 4, 5]


# --------------------------------------------------------------------------
# int4 gs64 storage: unpack, quantiser.
# --------------------------------------------------------------------------

def test_unpack_all_bytes():
    for b in range(256):
        row = np.array([b], np.uint8)
        lo, hi = b & 0xF, b >> 4
        assert oracle.unpack_code(row, 0) == (lo ^ 8) - 8
        assert oracle.unpack_code(row, 1) == (hi ^ 8) - 8
        assert -8 <= oracle.unpack_code(row, 0) <= 7


def test_unpack_matches_independent_quantiser():
    """Codes written by the generator decode to the codes a numpy quantiser
    computes from the same draws (s = absmax/7, q = rint(w/s) clamped)."""
    rows, cols = 16, 256
    tg = synth.tag(0, synth.KIND_GATE, 3)
    w = synth.normal_matrix(1, tg, rows, cols, 0.02)
    codes, scales = synth.quant_matrix(1, tg, rows, cols, 0.02)
    g = w.reshape(rows, cols // 64, 64)
    s = (np.abs(g).max(axis=2) / np.float32(7)).astype(np.float32)
    assert np.array_equal(s, scales)
    q = np.clip(np.rint(g / s[:, :, None]), -8, 7).astype(np.int32).reshape(rows, cols)
    for r in range(rows):
        dec = [oracle.unpack_code(codes[r], c) for c in range(cols)]
        assert dec == q[r].tolist()


def test_quantiser_properties():
    rows, cols = 64, 512
    tg = synth.tag(2, synth.KIND_DOWN, 1)
    w = synth.normal_matrix(9, tg, rows, cols, 0.02).astype(np.float64)
    codes, scales = synth.quant_matrix(9, tg, rows, cols, 0.02)
    lo = (codes & 0xF).astype(np.int32)
    hi = (codes >> 4).astype(np.int32)
    q = np.empty((rows, cols), np.int32)
    q[:, 0::2] = (lo ^ 8) - 8
    q[:, 1::2] = (hi ^ 8) - 8
    s = np.repeat(scales.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(w - q * s) <= s / 2 * (1 + 1e-6))
    assert q.min() >= -8 and q.max() <= 7
    # crafted groups: all zero -> s = 0, q = 0; -8 appears only via clamping
    wz = np.zeros((1, 64), np.float32)
    cz, sz = synth.quantize_rows(wz)
    assert sz[0, 0] == 0.0 and np.all(cz == 0)


# --------------------------------------------------------------------------
# Expert FFN and combine.
# --------------------------------------------------------------------------

def _dequant(codes, scales):
    lo = (codes & 0xF).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    q = np.empty((codes.shape[0], codes.shape[1] * 2), np.float64)
    q[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    q[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    return q * np.repeat(scales.astype(np.float64), 64, axis=1)


def _ffn_numpy(t, x):
    wg, wu, wd = _dequant(t["gate_q"], t["gate_s"]), _dequant(t["up_q"], t["up_s"]), _dequant(t["down_q"], t["down_s"])
    x = x.astype(np.float64)
    g, u = wg @ x, wu @ x
    return wd @ (g / (1.0 + np.exp(-g)) * u)


def test_expert_ffn_closed_form():
    """All gate codes 1, up codes 2, down codes -3, scales 0.5, x = 0.01:
    g = 0.5*h*0.01, u = 2*g, m = silu(g)*u, y_r = -1.5 * I * m."""
    h, I = 128, 64
    t = dict(gate_q=np.full((I, h // 2), 0x11, np.uint8), gate_s=np.full((I, h // 64), 0.5, np.float32),
             up_q=np.full((I, h // 2), 0x22, np.uint8), up_s=np.full((I, h // 64), 0.5, np.float32),
             down_q=np.full((h, I // 2), 0xDD, np.uint8), down_s=np.full((h, I // 64), 0.5, np.float32))
    x = np.full(h, 0.01, np.float32)
    xs = float(np.float32(0.01)) * h
    g = 0.5 * xs
    u = 2 * g
    m = g / (1 + math.exp(-g)) * u
    y = oracle.expert_ffn(t, x)
    assert np.allclose(y, -1.5 * I * m, rtol=1e-13, atol=0)


def test_expert_ffn_matches_numpy_float64():
    shape = synth.TINY
    t = synth.expert(shape, 5, 2)
    x = synth.hidden(shape, 5, 3)
    for r in range(3):
        assert np.allclose(oracle.expert_ffn(t, x[r]), _ffn_numpy(t, x[r]), rtol=1e-12, atol=1e-15)


def test_single_expert_layer_is_scaled_swiglu():
    """Textbook case E = 1, k = 1: the weight is rsf exactly, so
    out = rsf * FFN(x) + FFN_shared(x)."""
    shape = synth.LayerShape(hidden=128, n_experts=1, top_k=1, inter=192, n_shared=1, rsf=2.5, bias_sigma=0.0)
    wr, b = synth.router(shape, 3)
    routed = synth.routed_tables(shape, 3)
    sh = synth.shared_tables(shape, 3)
    x = synth.hidden(shape, 3, 5)
    out, idx, w = oracle.forward(shape, wr, b, routed, sh, x)
    assert np.all(idx == 0) and np.all(w == np.float32(2.5))
    t0 = {k: v[0] for k, v in routed.items()}
    for r in range(5):
        ref = 2.5 * _ffn_numpy(t0, x[r]) + _ffn_numpy(sh, x[r])
        assert np.allclose(out[r], ref, rtol=2e-7, atol=1e-7 * np.abs(ref).max())


@pytest.mark.parametrize("shape_kw", [dict(hidden=64, n_experts=8, inter=128, n_shared=1, rsf=1.0),
                                      dict(hidden=128, n_experts=6, inter=64, n_shared=0, rsf=2.5)])
def test_forced_all_experts_equals_dense_mixture(shape_kw):
    """k = E with zero bias: every expert is selected, so the dispatched,
    combined output equals the dense mixture sum_e (s_e / sum s) rsf FFN_e(x)
    + FFN_shared(x), here computed with numpy float64 and no grouping."""
    E = shape_kw["n_experts"]
    shape = synth.LayerShape(top_k=E, bias_sigma=0.0, **shape_kw)
    wr, b = synth.router(shape, 21)
    routed = synth.routed_tables(shape, 21)
    sh = synth.shared_tables(shape, 21)
    x = synth.hidden(shape, 21, 6)
    out, idx, w = oracle.forward(shape, wr, b, routed, sh, x)
    logits = x.astype(np.float64) @ wr.astype(np.float64)
    s = 1.0 / (1.0 + np.exp(-logits))
    for t in range(x.shape[0]):
        mix = np.zeros(shape.hidden)
        for e in range(E):
            te = {k: v[e] for k, v in routed.items()}
            mix += s[t, e] / s[t].sum() * shape.rsf * _ffn_numpy(te, x[t])
        if shape.n_shared:
            mix += _ffn_numpy(sh, x[t])
        assert np.allclose(out[t], mix, rtol=1e-5, atol=1e-5 * np.abs(mix).max())


def test_forward_tokens_are_independent():
    """Routing and FFN act per token: a permuted, duplicated batch gives the
    permuted, duplicated outputs bit for bit."""
    shape = synth.TINY
    wr, b = synth.router(shape, 4)
    routed = synth.routed_tables(shape, 4)
    sh = synth.shared_tables(shape, 4)
    x = synth.hidden(shape, 4, 5)
    out, idx, w = oracle.forward(shape, wr, b, routed, sh, x)
    perm = [3, 0, 0, 4, 2, 1, 3]
    out2, idx2, w2 = oracle.forward(shape, wr, b, routed, sh, x[perm])
    assert np.array_equal(out2, out[perm]) and np.array_equal(idx2, idx[perm]) and np.array_equal(w2, w[perm])


def test_forward_rejects_bad_k():
    shape = synth.LayerShape(hidden=64, n_experts=4, top_k=5, inter=64, n_shared=0, rsf=1.0, bias_sigma=0.0)
    wr, b = synth.router(shape, 1)
    routed = synth.routed_tables(shape, 1)
    with pytest.raises(ValueError, match="-2"):
        oracle.forward(shape, wr, b, routed, None, synth.hidden(shape, 1, 2))


@pytest.mark.parametrize("k_use,top_p", [(8, 0.7), (3, 1.0), (5, 0.5)])
def test_forward_with_routing_limits_equals_mixture_of_kept(k_use, top_p):
    """With routing limits the output is the mixture of the kept experts
    only, with the kept weights, plus the shared expert: computed here with
    numpy float64 per token, no grouping; dropped slots add nothing."""
    shape = synth.LayerShape(hidden=128, n_experts=16, top_k=8, inter=64, n_shared=1, rsf=2.5, bias_sigma=0.05)
    wr, b = synth.router(shape, 23)
    routed = synth.routed_tables(shape, 23)
    sh = synth.shared_tables(shape, 23)
    x = synth.hidden(shape, 23, 5)
    out, idx, w = oracle.forward(shape, wr, b, routed, sh, x, k_use=k_use, top_p=top_p)
    ri, rw = oracle.route(shape, wr, b, x, k_use=k_use, top_p=top_p)
    assert np.array_equal(idx, ri) and np.array_equal(w, rw)
    assert np.all((idx >= 0).sum(axis=1) <= k_use)
    for t in range(x.shape[0]):
        mix = _ffn_numpy(sh, x[t])
        for j in range(shape.top_k):
            if idx[t, j] >= 0:
                te = {kk: v[idx[t, j]] for kk, v in routed.items()}
                mix = mix + float(w[t, j]) * _ffn_numpy(te, x[t])
        assert np.allclose(out[t], mix, rtol=1e-6, atol=1e-6 * np.abs(mix).max())


# --------------------------------------------------------------------------
# int8 tables with one scale per row (the MTP head's format).
# --------------------------------------------------------------------------

def test_int8_code_all_bytes():
    """Every byte reads as its two's-complement value (numpy's int8 view is
    the independent reference)."""
    row = np.arange(256, dtype=np.uint8)
    want = row.view(np.int8).astype(int).tolist()
    assert [oracle.int8_code(row, c) for c in range(256)] == want


def test_int8_quantiser_properties():
    rng = np.random.default_rng(12)
    w = (0.02 * rng.standard_normal((40, 192))).astype(np.float32)
    w[3] = 0.0
    codes, scales = synth.quantize_rows_i8(w)
    q = codes.view(np.int8).astype(np.float64)
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(scales[3] == 0) and np.all(q[3] == 0)
    s = scales.astype(np.float64)[:, None]
    assert np.all(np.abs(w - q * s) <= s / 2 * (1 + 1e-6) + 1e-30)
    # the row's largest weight maps to +-127
    nz = np.arange(40) != 3
    assert np.all(np.abs(q[nz]).max(axis=1) == 127)


def _dequant_i8(codes, scales):
    return codes.view(np.int8).astype(np.float64) * scales.astype(np.float64)[:, None]


def _ffn_numpy_i8(t, x):
    wg, wu, wd = _dequant_i8(t["gate_q"], t["gate_s"]), _dequant_i8(t["up_q"], t["up_s"]), _dequant_i8(t["down_q"], t["down_s"])
    x = x.astype(np.float64)
    g, u = wg @ x, wu @ x
    return wd @ (g / (1.0 + np.exp(-g)) * u)


def test_int8_expert_ffn_closed_form():
    """Gate codes 3, up codes -2, down codes 5 (every byte), row scales 0.25,
    x = 0.01: g = 0.75 * h * 0.01, u = -2 g / 3, m = silu(g) u,
    y_r = 1.25 * I * m."""
    h, I = 128, 64
    t = dict(gate_q=np.full((I, h), 3, np.uint8), gate_s=np.full(I, 0.25, np.float32),
             up_q=np.full((I, h), 254, np.uint8), up_s=np.full(I, 0.25, np.float32),
             down_q=np.full((h, I), 5, np.uint8), down_s=np.full(h, 0.25, np.float32))
    x = np.full(h, 0.01, np.float32)
    xs = float(np.float32(0.01)) * h
    g = 0.75 * xs
    u = -0.5 * xs
    m = g / (1 + math.exp(-g)) * u
    y = oracle.expert_ffn(t, x, weight_format=1)
    assert np.allclose(y, 1.25 * I * m, rtol=1e-13, atol=0)


def test_int8_expert_ffn_matches_numpy_float64():
    shape = synth.TINY_I8
    t = synth.expert(shape, 5, 2)
    assert t["gate_q"].shape == (shape.inter, shape.hidden) and t["gate_s"].shape == (shape.inter,)
    x = synth.hidden(shape, 5, 3)
    for r in range(3):
        assert np.allclose(oracle.expert_ffn(t, x[r], weight_format=1), _ffn_numpy_i8(t, x[r]), rtol=1e-12,
                           atol=1e-15)


def test_int8_all_codes_including_minus_128():
    """Random bytes (every code, -128 included) and random row scales."""
    rng = np.random.default_rng(13)
    h, I = 128, 64
    t = dict(gate_q=rng.integers(0, 256, (I, h), dtype=np.uint8), gate_s=rng.uniform(1e-4, 1e-3, I).astype(np.float32),
             up_q=rng.integers(0, 256, (I, h), dtype=np.uint8), up_s=rng.uniform(1e-4, 1e-3, I).astype(np.float32),
             down_q=rng.integers(0, 256, (h, I), dtype=np.uint8), down_s=rng.uniform(1e-4, 1e-3, h).astype(np.float32))
    x = rng.standard_normal(h).astype(np.float32)
    assert np.allclose(oracle.expert_ffn(t, x, weight_format=1), _ffn_numpy_i8(t, x), rtol=1e-12, atol=1e-15)


def test_int8_single_expert_layer_is_scaled_swiglu():
    shape = synth.LayerShape(hidden=128, n_experts=1, top_k=1, inter=192, n_shared=1, rsf=2.5, bias_sigma=0.0,
                             weight_format=synth.WEIGHTS_INT8_ROW)
    wr, b = synth.router(shape, 3)
    routed = synth.routed_tables(shape, 3)
    sh = synth.shared_tables(shape, 3)
    x = synth.hidden(shape, 3, 5)
    out, idx, w = oracle.forward(shape, wr, b, routed, sh, x)
    assert np.all(idx == 0) and np.all(w == np.float32(2.5))
    t0 = {k: v[0] for k, v in routed.items()}
    for r in range(5):
        ref = 2.5 * _ffn_numpy_i8(t0, x[r]) + _ffn_numpy_i8(sh, x[r])
        assert np.allclose(out[r], ref, rtol=2e-7, atol=1e-7 * np.abs(ref).max())


def test_int8_forced_all_experts_equals_dense_mixture():
    E = 6
    shape = synth.LayerShape(hidden=128, n_experts=E, inter=64, n_shared=1, rsf=2.5, top_k=E, bias_sigma=0.0,
                             weight_format=synth.WEIGHTS_INT8_ROW)
    wr, b = synth.router(shape, 24)
    routed = synth.routed_tables(shape, 24)
    sh = synth.shared_tables(shape, 24)
    x = synth.hidden(shape, 24, 4)
    out, _, _ = oracle.forward(shape, wr, b, routed, sh, x)
    s = 1.0 / (1.0 + np.exp(-(x.astype(np.float64) @ wr.astype(np.float64))))
    for t in range(4):
        mix = _ffn_numpy_i8(sh, x[t])
        for e in range(E):
            mix += s[t, e] / s[t].sum() * shape.rsf * _ffn_numpy_i8({k: v[e] for k, v in routed.items()}, x[t])
        assert np.allclose(out[t], mix, rtol=1e-5, atol=1e-5 * np.abs(mix).max())

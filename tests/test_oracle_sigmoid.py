"""Pins for the oracle's group-limited sigmoid routing
(oracle.grouped.route_sigmoid_grouped) and its forward.

Contract: ruDNN user guide (RUDA docs, German edition), section 10.
Pins, none of which reuses the oracle's own formulation:
* golden cases worked out by hand from the section (tests/golden);
* brute force by counting: a group is kept iff fewer than selected_groups
  groups beat it, an expert is chosen iff fewer than top_k eligible experts
  beat it, its slot is that count, and a top-two group score is the FP32
  sum of the pair of the group's experts whose (larger, smaller) values are
  lexicographically largest;
* one group, or every group selected, reduces to a stable descending sort
  (numpy) of the corrected values;
* the sigmoid against scipy's ``expit`` and its closed-form values;
* unrenormalised weights are the sigmoid of the chosen logits whatever the
  bias; renormalised weights sum to ``scale``;
* the option limits of the section;
* the forward equals a per-token sum over the chosen experts, and with
  identical experts the expert output times the summed weights; the
  token-by-token form agrees with the full forward.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle.fp import round_to
from oracle.grouped import (check_options, forward_sigmoid_grouped,
                            forward_sigmoid_tokens, route_sigmoid_grouped,
                            sigmoid_fp32)
from oracle.moe import expert_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "sigmoid_grouped_cases.json")


def _val(v):
    return {"nan": np.nan, "inf": np.inf, "-inf": -np.inf}.get(v, v)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _logits_of(case):
    if "logits" in case:
        return np.array([[_val(v) for v in case["logits"]]], dtype=np.float32)
    p = np.array(case["p"], dtype=np.float64)
    return np.log(p / (1.0 - p)).astype(np.float32)[None, :]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_golden_cases(case):
    fmt = case.get("fmt", "f32")
    lg = _logits_of(case)
    if fmt != "f32":
        lg = round_to(lg.astype(np.float64), fmt)
    bias = (None if "bias" not in case
            else np.array([_val(v) for v in case["bias"]], dtype=np.float32))
    idx, w = route_sigmoid_grouped(lg, bias, case["k"], case["groups"],
                                   case["selected_groups"],
                                   case["group_top_two"], case["renormalize"],
                                   case["scale"], fmt)
    assert idx[0].tolist() == case["idx"]
    for got, want in zip(w[0], case["w"]):
        if want is None:
            assert np.isnan(got)
        elif case.get("exact"):
            assert got == want
        else:
            assert abs(got - want) <= 1e-6, (got, want)


# ---------------------------------------------------------------------------
# brute force by counting
# ---------------------------------------------------------------------------

def _beats(a, i, b, j):
    """(a, id i) ranks before (b, id j): larger value, then smaller id."""
    return a > b or (a == b and i < j)


def _brute(row, bias, k, groups, sg, top_two):
    E = len(row)
    size = E // groups
    s = expit(row.astype(np.float64)).astype(np.float32)
    c = [np.float32(s[e] + bias[e]) for e in range(E)]
    if any(np.isnan(v) for v in c):
        return list(range(k))
    gsc = []
    for g in range(groups):
        vals = c[g * size:(g + 1) * size]
        if top_two:
            # the pair whose (larger, smaller) values are largest, summed
            pair = max((max(vals[a], vals[b]), min(vals[a], vals[b]))
                       for a, b in itertools.combinations(range(size), 2))
            with np.errstate(invalid="ignore"):
                gsc.append(np.float32(pair[0] + pair[1]))
        else:
            gsc.append(max(vals))
    if any(np.isnan(v) for v in gsc):
        return list(range(k))
    kept = [g for g in range(groups)
            if sum(_beats(gsc[h], h, gsc[g], g) for h in range(groups)) < sg]
    elig = [e for e in range(E) if e // size in kept]
    slot = {}
    for e in elig:
        n = sum(_beats(c[f], f, c[e], e) for f in elig)
        if n < k:
            slot[n] = e
    return [slot[j] for j in range(k)]


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


@pytest.mark.parametrize("seed", range(5))
def test_brute_force_small(seed):
    rng = np.random.default_rng(seed)
    for _ in range(30):
        E = int(rng.integers(1, 9))
        T = int(rng.integers(1, 4))
        # a coarse grid of logits and biases -> many equal scores
        lg = (rng.integers(-2, 3, size=(T, E)) * 0.5).astype(np.float32)
        bias = (rng.integers(-1, 2, size=E) * 0.25).astype(np.float32)
        for groups in _divisors(E):
            size = E // groups
            for sg in range(1, groups + 1):
                for top_two in ((False, True) if size >= 2 else (False,)):
                    for k in sorted({1, sg * size, max(1, sg * size // 2)}):
                        idx, _ = route_sigmoid_grouped(
                            lg, bias, k, groups, sg, top_two, False, 1.0,
                            "f32")
                        for t in range(T):
                            want = _brute(lg[t], bias, k, groups, sg, top_two)
                            assert idx[t].tolist() == want, (lg[t], bias, k,
                                                             groups, sg,
                                                             top_two)


def test_brute_force_with_special_values():
    rng = np.random.default_rng(11)
    specials = np.array([np.inf, -np.inf, np.nan, 0.0, 30.0, -30.0, -120.0],
                        dtype=np.float32)
    for _ in range(300):
        E = int(rng.integers(2, 9))
        lg = rng.choice(specials[:-1] if rng.random() < 0.7 else specials,
                        size=(1, E)).astype(np.float32)
        bias = rng.choice(np.array([0.0, np.inf, -np.inf, 0.5],
                                   dtype=np.float32), size=E)
        groups = int(rng.choice(_divisors(E)))
        size = E // groups
        sg = int(rng.integers(1, groups + 1))
        top_two = bool(size >= 2 and rng.random() < 0.5)
        k = int(rng.integers(1, sg * size + 1))
        idx, w = route_sigmoid_grouped(lg, bias, k, groups, sg, top_two,
                                       False, 1.0, "f32")
        assert idx[0].tolist() == _brute(lg[0], bias, k, groups, sg, top_two)


# ---------------------------------------------------------------------------
# reductions to library routines and closed forms
# ---------------------------------------------------------------------------

def test_sigmoid_matches_expit_and_closed_forms():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 8,
                        np.linspace(-110, 40, 4001)]).astype(np.float32)
    got = sigmoid_fp32(x)
    want = expit(x.astype(np.float64)).astype(np.float32)
    # both are within a few float64 ulps of the exact sigmoid before the
    # float32 rounding, so they agree unless a value lies that close to a
    # float32 rounding boundary
    assert (got == want).mean() > 0.999999
    assert np.all(np.abs(got.astype(np.float64) - want) <=
                  np.spacing(np.abs(want)))
    assert sigmoid_fp32(np.float32(0.0)) == np.float32(0.5)
    assert sigmoid_fp32(np.float32(np.inf)) == np.float32(1.0)
    assert sigmoid_fp32(np.float32(-np.inf)) == np.float32(0.0)
    assert np.isnan(sigmoid_fp32(np.float32(np.nan)))
    # sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4 (the float32 logit is off by
    # under half an ulp, which moves sigma by far less than a float32 ulp)
    assert sigmoid_fp32(np.float32(math.log(3))) == np.float32(0.75)
    assert sigmoid_fp32(np.float32(-math.log(3))) == np.float32(0.25)
    # monotone
    xs = np.sort(x)
    assert np.all(np.diff(sigmoid_fp32(xs).astype(np.float64)) >= 0)


@pytest.mark.parametrize("with_bias", [False, True])
def test_one_group_is_a_stable_descending_sort(with_bias):
    rng = np.random.default_rng(7)
    T, E = 50, 24
    lg = (rng.integers(-6, 7, size=(T, E)) * 0.25).astype(np.float32)
    bias = ((rng.integers(-2, 3, size=E) * 0.125).astype(np.float32)
            if with_bias else None)
    b = np.zeros(E, np.float32) if bias is None else bias
    for k in (1, 5, E):
        idx1, w1 = route_sigmoid_grouped(lg, bias, k, 1, 1, False, False,
                                         1.0, "f32")
        # all groups selected: the group limit is inactive
        idx2, w2 = route_sigmoid_grouped(lg, bias, k, 6, 6, True, False,
                                         1.0, "f32")
        for t in range(T):
            c = (expit(lg[t].astype(np.float64)).astype(np.float32)
                 + b).astype(np.float32)
            want = np.argsort(-c.astype(np.float64), kind="stable")[:k]
            assert idx1[t].tolist() == want.tolist()
            assert idx2[t].tolist() == want.tolist()
        assert np.array_equal(w1, w2)


def test_weights_are_sigmoid_of_chosen_logits_whatever_the_bias():
    rng = np.random.default_rng(9)
    T, E = 40, 32
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for bias_std in (0.0, 0.3, 3.0):
        bias = (rng.standard_normal(E) * bias_std).astype(np.float32)
        idx, w = route_sigmoid_grouped(lg, bias, 6, 8, 3, True, False, 1.0,
                                       "f32")
        for t in range(T):
            want = expit(lg[t, idx[t]].astype(np.float64)).astype(np.float32)
            assert np.all(np.abs(w[t] - want) <= np.spacing(want))


@pytest.mark.parametrize("scale", [1.0, 2.5, 0.125])
def test_renormalised_weights_sum_to_scale(scale):
    rng = np.random.default_rng(13)
    T, E = 40, 64
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = route_sigmoid_grouped(lg, None, 8, 8, 4, True, True, scale,
                                   "f32")
    assert np.allclose(w.sum(axis=1), scale, rtol=1e-6, atol=0)


def test_option_limits():
    ok = dict(E=64, k=8, groups=8, selected_groups=4, group_top_two=True,
              scale=2.5)
    check_options(**ok)
    check_options(E=1024, k=64, groups=128, selected_groups=128,
                  group_top_two=True, scale=1e30)
    check_options(E=1, k=1, groups=1, selected_groups=1, group_top_two=False,
                  scale=1.0)
    bad = [dict(E=0), dict(E=1025, groups=1, selected_groups=1),
           dict(groups=0), dict(groups=7), dict(E=256, groups=256),
           dict(selected_groups=0), dict(selected_groups=9), dict(k=0),
           dict(k=65), dict(k=33, selected_groups=4),
           dict(E=8, groups=8, k=1, selected_groups=1),
           dict(scale=0.0), dict(scale=-1.0), dict(scale=math.inf),
           dict(scale=math.nan)]
    for b in bad:
        args = dict(ok, **b)
        with pytest.raises(ValueError):
            check_options(**args)
    # k equal to the kept experts is allowed
    check_options(E=64, k=32, groups=8, selected_groups=4,
                  group_top_two=False, scale=1.0)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def _small_layer(rng, T, H, I, E):
    x = rng.standard_normal((T, H)).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    wg = (rng.standard_normal((E, I, H)) / math.sqrt(H)).astype(np.float32)
    wu = (rng.standard_normal((E, I, H)) / math.sqrt(H)).astype(np.float32)
    wd = (rng.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32)
    return x, lg, wg, wu, wd


def test_forward_is_a_per_token_sum():
    rng = np.random.default_rng(17)
    T, H, I, E = 4, 8, 12, 8
    x, lg, wg, wu, wd = _small_layer(rng, T, H, I, E)
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    r = forward_sigmoid_grouped(x, lg, bias, wg, wu, wd, 3, 4, 2, True, True,
                                2.5, "f32")
    for t in range(T):
        acc = np.zeros(H)
        for j in range(3):
            e = int(r["idx"][t, j])
            y = expert_rows(x[t].astype(np.float64)[None, :], e,
                            wg[e].astype(np.float64),
                            wu[e].astype(np.float64),
                            wd[e].astype(np.float64), "f32")[0]
            acc = acc + r["w"][t, j] * y
        assert np.array_equal(r["out"][t], round_to(acc, "f32"))


def test_forward_with_identical_experts():
    rng = np.random.default_rng(19)
    T, H, I, E = 6, 8, 16, 8
    x, lg, wg, wu, wd = _small_layer(rng, T, H, I, E)
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    r = forward_sigmoid_grouped(x, lg, None, wg, wu, wd, 4, 4, 3, False,
                                False, 1.0, "f32")
    y = expert_rows(x.astype(np.float64), 0, wg[0].astype(np.float64),
                    wu[0].astype(np.float64), wd[0].astype(np.float64), "f32")
    want = round_to(r["w"].sum(axis=1)[:, None] * y, "f32")
    assert np.allclose(r["out"], want, rtol=1e-6, atol=1e-7)


def test_token_by_token_forward_matches_full_forward():
    rng = np.random.default_rng(23)
    T, H, I, E = 7, 8, 12, 16
    x, lg, wg, wu, wd = _small_layer(rng, T, H, I, E)
    bias = (rng.standard_normal(E) * 0.2).astype(np.float32)
    full = forward_sigmoid_grouped(x, lg, bias, wg, wu, wd, 4, 4, 2, True,
                                   True, 2.5, "f32")
    tokens = [0, 3, 6]
    idx, w, out = forward_sigmoid_tokens(x, lg, bias, wg, wu, wd, 4, 4, 2,
                                         True, True, 2.5, "f32", tokens)
    assert np.array_equal(idx, full["idx"][tokens])
    assert np.array_equal(w, full["w"][tokens])
    assert np.allclose(out, full["out"][tokens], rtol=1e-6, atol=1e-7)

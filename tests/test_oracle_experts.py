"""Pins for the oracle's expert, combine and whole-forward steps.

Expert stage: docs.rs "ruDNN 0.1.25 source, src/moe/experts.rs",
SwiGluExperts::new (gate/up [E,I,H], down [E,H,I], bias free) and
forward_dispatched_with_strategy (gate product, up product, the swiglu kernel
writing SiLU(gate)*up into gate's storage, then the down product).  Combine:
ruDNN user guide (RUDA docs), section 6 (weights applied while merging).

Pins (none reuses the oracle's vectorised code):
* brute force with Python loops over every index and math.fsum sums, at
  T <= 4, H=3, I=5 (non-square so a transposed weight fails), all k, both
  renormalisation settings, every format: must agree bit for bit;
* E = 1 reduces to a dense SwiGLU MLP, checked with torch float64 matmuls;
* H = I = 1 scalar closed form;
* k = 1 with renormalisation: the output is the expert row, bit for bit;
* identical experts with renormalisation: the output does not depend on
  the routing (the weights sum to one);
* the activation rows (``experts(..., with_act=True)``) equal the loops'
  SiLU(gate) * up bit for bit, every format;
* the token-by-token forward (``forward_tokens``, the checker behind the
  full-size end-to-end tests) equals the loops directly, and the full
  forward restricted to its tokens bit for bit, for every format, k in
  {1, 2, E}, both renormalisation settings, poisoned rows and unsorted,
  repeated token lists.
"""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle.fp import round_to
from oracle.moe import (combine, dispatch, experts, forward, forward_tokens,
                        route)


def _rnd(v, fmt):
    return float(round_to(np.array([v]), fmt)[0])


def _mlp_loops(x, wg, wu, wd, fmt, with_act=False):
    """One token through one expert with explicit loops.
    wg, wu: nested lists [I][H]; wd: [H][I].  With ``with_act`` also the
    activation row a (the experts page's stored SwiGLU result)."""
    H, I = len(x), len(wg)
    g = [_rnd(math.fsum(x[h] * wg[i][h] for h in range(H)), fmt)
         for i in range(I)]
    u = [_rnd(math.fsum(x[h] * wu[i][h] for h in range(H)), fmt)
         for i in range(I)]
    a = []
    for i in range(I):
        try:
            sig = 1.0 / (1.0 + math.exp(-g[i]))
        except OverflowError:
            sig = 0.0
        a.append(_rnd(g[i] * sig * u[i], fmt))
    y = [_rnd(math.fsum(a[i] * wd[h][i] for i in range(I)), fmt)
         for h in range(H)]
    return (y, a) if with_act else y


def _case(rng, T, H, I, E, fmt):
    x = round_to(rng.standard_normal((T, H)), fmt)
    lg = round_to(rng.integers(-4, 5, size=(T, E)) * 0.5
                  + rng.standard_normal((T, E)) * 0.1, fmt)
    wg = round_to(rng.standard_normal((E, I, H)) / math.sqrt(H), fmt)
    wu = round_to(rng.standard_normal((E, I, H)) / math.sqrt(H), fmt)
    wd = round_to(rng.standard_normal((E, H, I)) / math.sqrt(I), fmt)
    return x, lg, wg, wu, wd


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_forward_brute_force_tiny(fmt):
    rng = np.random.default_rng({"f32": 1, "f16": 2, "bf16": 3}[fmt])
    H, I, E = 3, 5, 4
    for T in (1, 2, 4):
        x, lg, wg, wu, wd = _case(rng, T, H, I, E, fmt)
        for k, renorm in itertools.product(range(1, E + 1), (False, True)):
            res = forward(x, lg, wg, wu, wd, k, renorm, fmt)
            idx, w = res["idx"], res["w"]
            for t in range(T):
                acc = []
                for j in range(k):
                    e = int(idx[t, j])
                    y = _mlp_loops(list(x[t]), wg[e].tolist(), wu[e].tolist(),
                                   wd[e].tolist(), fmt)
                    acc.append([w[t, j] * v for v in y])
                want = [_rnd(math.fsum(col), fmt) for col in zip(*acc)]
                assert res["out"][t].tolist() == want, (T, k, renorm, t)


def test_single_expert_is_dense_swiglu_mlp():
    rng = np.random.default_rng(21)
    T, H, I = 12, 64, 96
    x, lg, wg, wu, wd = _case(rng, T, H, I, 1, "f32")
    res = forward(x, lg, wg, wu, wd, 1, True, "f32")
    assert np.all(res["w"] == 1.0)
    X = torch.from_numpy(x)
    g = torch.from_numpy(round_to((X @ torch.from_numpy(wg[0]).T).numpy(),
                                  "f32"))
    u = torch.from_numpy(round_to((X @ torch.from_numpy(wu[0]).T).numpy(),
                                  "f32"))
    a = torch.from_numpy(round_to((torch.nn.functional.silu(g) * u).numpy(),
                                  "f32"))
    y = round_to((a @ torch.from_numpy(wd[0]).T).numpy(), "f32")
    np.testing.assert_allclose(res["out"], y, rtol=2e-7, atol=0)


def test_scalar_closed_form():
    # H = I = 1: y = rnd(rnd(silu(rnd(x*wg)) * rnd(x*wu))* wd)
    fmt = "bf16"
    for xv, g, u, d in [(1.5, 0.75, -2.0, 0.5), (-3.0, 1.25, 0.375, -1.0),
                        (0.0, 1.0, 1.0, 1.0), (2.0, -40.0, 3.0, 1.0)]:
        x = np.array([[xv]])
        wg = np.array([[[g]]])
        wu = np.array([[[u]]])
        wd = np.array([[[d]]])
        gg, uu = _rnd(xv * g, fmt), _rnd(xv * u, fmt)
        a = _rnd(gg / (1.0 + math.exp(-gg)) * uu, fmt)
        want = _rnd(a * d, fmt)
        y = experts(x, np.array([0, 1]), wg, wu, wd, fmt)
        assert y[0, 0] == want


def test_k1_renormalised_combine_is_identity():
    rng = np.random.default_rng(4)
    T, H, I, E = 20, 8, 12, 5
    x, lg, wg, wu, wd = _case(rng, T, H, I, E, "bf16")
    res = forward(x, lg, wg, wu, wd, 1, True, "bf16")
    tr = res["dispatch"]["token_row"][:, 0]
    np.testing.assert_array_equal(res["out"], res["y"][tr])


def test_identical_experts_ignore_routing():
    rng = np.random.default_rng(8)
    T, H, I, E = 16, 8, 12, 6
    x, lg, wg, wu, wd = _case(rng, T, H, I, E, "f32")
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    single = experts(x, np.array([0, T]), wg[:1], wu[:1], wd[:1], "f32")
    for k in (1, 3, 6):
        res = forward(x, lg, wg, wu, wd, k, True, "f32")
        np.testing.assert_allclose(res["out"], single, rtol=k * 2.0 ** -22,
                                   atol=1e-30)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(12)
    T, H, I, E = 30, 8, 12, 4
    x, lg, wg, wu, wd = _case(rng, T, H, I, E, "f16")
    idx, w = route(lg, 2, True, "f16")
    d = dispatch(x, idx, E)
    full = experts(d["xd"], d["offsets"], wg, wu, wd, "f16")
    rows = [59, 0, 17, 33]
    part = experts(d["xd"], d["offsets"], wg, wu, wd, "f16", rows=rows)
    np.testing.assert_array_equal(part, full[rows])
    out = combine(full, w, d["token_row"], "f16")
    out3 = combine(full, w, d["token_row"], "f16", tokens=[3, 7])
    np.testing.assert_array_equal(out3, out[[3, 7]])


def test_poisoned_row_gives_nan_output_only_there():
    rng = np.random.default_rng(13)
    T, H, I, E = 6, 4, 6, 3
    x, lg, wg, wu, wd = _case(rng, T, H, I, E, "f16")
    lg[2, 1] = np.nan
    lg[4] = -np.inf
    res = forward(x, lg, wg, wu, wd, 2, True, "f16")
    bad = np.isnan(res["out"]).all(axis=1)
    assert bad.tolist() == [False, False, True, False, True, False]
    assert not np.isnan(res["out"][~bad]).any()


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_activation_rows_brute_force(fmt):
    rng = np.random.default_rng({"f32": 31, "f16": 32, "bf16": 33}[fmt])
    T, H, I, E, k = 6, 3, 5, 3, 2
    x, lg, wg, wu, wd = _case(rng, T, H, I, E, fmt)
    idx, _ = route(lg, k, True, fmt)
    d = dispatch(x, idx, E)
    y, act = experts(d["xd"], d["offsets"], wg, wu, wd, fmt, with_act=True)
    assert act.shape == (T * k, I)
    for r in range(T * k):
        e = int(d["row_expert"][r])
        yl, al = _mlp_loops(list(d["xd"][r]), wg[e].tolist(), wu[e].tolist(),
                            wd[e].tolist(), fmt, with_act=True)
        assert act[r].tolist() == al, (fmt, r)
        assert y[r].tolist() == yl, (fmt, r)
    # a row subset returns the same activation rows, in the order asked
    rows = [7, 0, 11, 3]
    ys, acts = experts(d["xd"], d["offsets"], wg, wu, wd, fmt, rows=rows,
                       with_act=True)
    np.testing.assert_array_equal(acts, act[rows])
    np.testing.assert_array_equal(ys, y[rows])


def _poison(lg):
    lg = lg.copy()
    lg[1, 0] = np.nan
    lg[3, 2] = np.inf
    lg[4] = -np.inf
    return lg


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_forward_tokens_brute_force(fmt):
    """forward_tokens against explicit loops: route, each slot's expert on
    the token row, the weighted sum in slot order rounded once."""
    rng = np.random.default_rng({"f32": 41, "f16": 42, "bf16": 43}[fmt])
    T, H, I, E = 6, 3, 5, 4
    x, lg, wg, wu, wd = _case(rng, T, H, I, E, fmt)
    lg = _poison(lg)
    tokens = [5, 0, 3, 3, 1, 4]
    for k, renorm in itertools.product((1, 2, E), (False, True)):
        idx, w, out = forward_tokens(x, lg, wg, wu, wd, k, renorm, fmt,
                                     tokens)
        ridx, rw = route(lg[tokens], k, renorm, fmt)
        np.testing.assert_array_equal(idx, ridx)
        np.testing.assert_array_equal(w, rw)
        for n, t in enumerate(tokens):
            acc = []
            for j in range(k):
                e = int(idx[n, j])
                y = _mlp_loops(list(x[t]), wg[e].tolist(), wu[e].tolist(),
                               wd[e].tolist(), fmt)
                acc.append([w[n, j] * v for v in y])
            if np.isnan(w[n]).any():
                assert np.isnan(out[n]).all(), (k, renorm, t)
                continue
            want = [_rnd(math.fsum(col), fmt) for col in zip(*acc)]
            assert out[n].tolist() == want, (fmt, k, renorm, t)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_forward_tokens_equals_full_forward(fmt):
    rng = np.random.default_rng({"f32": 51, "f16": 52, "bf16": 53}[fmt])
    T, H, I, E = 9, 8, 12, 5
    x, lg, wg, wu, wd = _case(rng, T, H, I, E, fmt)
    lg = _poison(lg)
    tokens = [8, 2, 2, 0, 4, 1, 3, 7]   # unsorted, one repeated
    for k, renorm in itertools.product((1, 2, E), (False, True)):
        full = forward(x, lg, wg, wu, wd, k, renorm, fmt)
        idx, w, out = forward_tokens(x, lg, wg, wu, wd, k, renorm, fmt,
                                     tokens)
        np.testing.assert_array_equal(idx, full["idx"][tokens])
        np.testing.assert_array_equal(w, full["w"][tokens])
        np.testing.assert_array_equal(out, full["out"][tokens])
        assert np.isnan(out[[tokens.index(t) for t in (1, 3, 4)]]).all()

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
  the routing (the weights sum to one).
"""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle.fp import round_to
from oracle.moe import combine, dispatch, experts, forward, route


def _rnd(v, fmt):
    return float(round_to(np.array([v]), fmt)[0])


def _mlp_loops(x, wg, wu, wd, fmt):
    """One token through one expert with explicit loops.
    wg, wu: nested lists [I][H]; wd: [H][I]."""
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
    return [_rnd(math.fsum(a[i] * wd[h][i] for i in range(I)), fmt)
            for h in range(H)]


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

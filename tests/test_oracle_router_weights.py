"""Pins for the oracle's router weights for a fixed selection and their
logits gradient (oracle.router_weights).

Contract: ruDNN user guide (RUDA docs, German edition), section 12.
Pins, none of which reuses the oracle's worked-out gradient:
* torch autograd in float64 on the weights written as the section defines
  them (softmax or sigmoid, gather, optional renormalisation, scale);
* central finite differences of the weights in float64;
* closed forms for two experts and for one slot;
* invariants: a softmax gradient row sums to zero; renormalised weights sum
  to ``scale``; one renormalised slot weighs ``scale`` with zero gradient;
* gather semantics of repeated indices, invalid indices, NaN and infinite
  logits, and the option limits.
"""

import math

import numpy as np
import pytest
import torch

from oracle.router_weights import (check_options, selected_router_backward,
                                   selected_router_weights)

LN3 = math.log(3.0)


def _torch_weights(x, ind, scoring, renorm, scale):
    """The section's definition in torch (float64, differentiable)."""
    s = torch.softmax(x, dim=-1) if scoring == "softmax" else torch.sigmoid(x)
    u = torch.gather(s, 1, ind)
    if renorm:
        u = u / u.sum(dim=1, keepdim=True)
    return scale * u


def _case(rng, T, E, k, repeats=False):
    x = rng.standard_normal((T, E)).astype(np.float32)
    if repeats:
        ind = rng.integers(0, E, size=(T, k))
    else:
        ind = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    g = rng.standard_normal((T, k)).astype(np.float32)
    return x, ind, g


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("repeats", [False, True])
def test_matches_torch_autograd(scoring, renorm, repeats):
    rng = np.random.default_rng(1 + 2 * renorm + 4 * repeats)
    T, E, k = 24, 12, 5
    x, ind, g = _case(rng, T, E, k, repeats)
    scale = 2.5
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    it = torch.tensor(ind, dtype=torch.int64)
    w_t = _torch_weights(xt, it, scoring, renorm, scale)
    (w_t * torch.tensor(g, dtype=torch.float64)).sum().backward()
    w = selected_router_weights(x, ind, scoring, renorm, scale, "f32")
    dx = selected_router_backward(x, ind, g, scoring, renorm, scale, "f32")
    want_w = w_t.detach().numpy()
    want_dx = xt.grad.numpy()
    assert np.allclose(w, want_w, rtol=1e-6, atol=0)
    # relative to each row's largest gradient entry (cancellation in the
    # exact formulas is below float32 rounding)
    tol = 1e-6 * np.abs(want_dx).max(axis=1, keepdims=True)
    assert np.all(np.abs(dx - want_dx) <= tol + 1e-30)
    if scoring == "sigmoid":
        sel = np.zeros((T, E), dtype=bool)
        np.put_along_axis(sel, ind, True, axis=1)
        assert np.all(dx[~sel] == 0.0)


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renorm", [False, True])
def test_matches_finite_differences(scoring, renorm):
    rng = np.random.default_rng(7)
    T, E, k = 4, 6, 3
    x, ind, g = _case(rng, T, E, k, repeats=True)
    x = x.astype(np.float64)
    scale = 0.75
    dx = selected_router_backward(x, ind, g, scoring, renorm, scale, "f32")

    def loss(xx):
        return (selected_router_weights(xx, ind, scoring, renorm, scale,
                                        "f32") * g).sum()

    # float64 weights for the differences: the same definition, unrounded
    def loss64(xx):
        out = 0.0
        for t in range(T):
            row = xx[t]
            if scoring == "softmax":
                q = np.exp(row - row.max())
                s = q / q.sum()
            else:
                s = 1.0 / (1.0 + np.exp(-row))
            u = s[ind[t]]
            if renorm:
                u = u / u.sum()
            out += (scale * u * g[t]).sum()
        return out

    h = 1e-6
    fd = np.zeros_like(x)
    for t in range(T):
        for e in range(E):
            xp, xm = x.copy(), x.copy()
            xp[t, e] += h
            xm[t, e] -= h
            fd[t, e] = (loss64(xp) - loss64(xm)) / (2 * h)
    assert np.allclose(dx, fd, rtol=1e-5, atol=1e-7)
    # and the FP32 weights are the float64 ones rounded
    assert abs(loss(x) - loss64(x)) <= 1e-6 * max(1.0, abs(loss64(x)))


def test_two_expert_closed_forms():
    x = np.array([[LN3, 0.0]], dtype=np.float32)     # softmax (3/4, 1/4)
    ind = np.array([[0]])
    w = selected_router_weights(x, ind, "softmax", False, 1.0, "f32")
    assert abs(w[0, 0] - 0.75) <= 1e-7
    dx = selected_router_backward(x, ind, np.ones((1, 1)), "softmax", False,
                                  1.0, "f32")
    # d p0 / d x = p0 * (delta - p) = (3/16, -3/16)
    assert np.allclose(dx[0], [0.1875, -0.1875], rtol=1e-6)
    # sigmoid at 0: weight 1/2, derivative 1/4, times scale
    x0 = np.zeros((1, 2), dtype=np.float32)
    w = selected_router_weights(x0, np.array([[1]]), "sigmoid", False, 2.5,
                                "f32")
    assert w[0, 0] == 1.25
    dx = selected_router_backward(x0, np.array([[1]]), np.ones((1, 1)),
                                  "sigmoid", False, 2.5, "f32")
    assert dx[0].tolist() == [0.0, 0.625]


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_invariants(scoring):
    rng = np.random.default_rng(3)
    T, E, k = 30, 16, 6
    x, ind, g = _case(rng, T, E, k)
    w = selected_router_weights(x, ind, scoring, True, 2.5, "f32")
    assert np.allclose(w.sum(axis=1), 2.5, rtol=1e-6)
    one = selected_router_weights(x, ind[:, :1], scoring, True, 2.5, "f32")
    assert np.all(one == 2.5)
    d1 = selected_router_backward(x, ind[:, :1], g[:, :1], scoring, True,
                                  2.5, "f32")
    assert np.all(np.abs(d1) <= 1e-7 * np.abs(g[:, :1]))
    if scoring == "softmax":
        for renorm in (False, True):
            dx = selected_router_backward(x, ind, g, scoring, renorm, 1.0,
                                          "f32")
            # softmax is invariant to a shift of the row
            assert np.all(np.abs(dx.sum(axis=1)) <=
                          1e-6 * np.abs(dx).sum(axis=1))
        # every expert selected once, renormalised: the softmax itself
        perm = np.stack([rng.permutation(E) for _ in range(T)])
        wa = selected_router_weights(x, perm, scoring, True, 1.0, "f32")
        wb = selected_router_weights(x, perm, scoring, False, 1.0, "f32")
        assert np.allclose(wa, wb, rtol=1e-6)


def test_repeated_indices_gather():
    x = np.array([[0.3, -1.2, 2.0]], dtype=np.float32)
    ind = np.array([[2, 2, 0]])
    w = selected_router_weights(x, ind, "softmax", False, 1.0, "f32")
    assert w[0, 0] == w[0, 1]
    wr = selected_router_weights(x, ind, "softmax", True, 1.0, "f32")
    p = np.exp(x[0].astype(np.float64))
    assert np.allclose(wr[0], [p[2] / (2 * p[2] + p[0])] * 2
                       + [p[0] / (2 * p[2] + p[0])], rtol=1e-6)


def test_invalid_indices_poison_the_row():
    x = np.zeros((4, 5), dtype=np.float32)
    for ind in (np.array([[0, 5]] * 4), np.array([[-1, 2]] * 4, np.int32),
                np.array([[0, 2**32 - 1]] * 4, np.uint32),
                np.array([[3, -(2**40)]] * 4, np.int64)):
        ind = ind.copy()
        ind[1] = [1, 2]                    # one valid row
        for scoring in ("softmax", "sigmoid"):
            w = selected_router_weights(x, ind, scoring, True, 1.0, "f32")
            dx = selected_router_backward(x, ind, np.ones((4, 2)), scoring,
                                          False, 1.0, "f32")
            for t in range(4):
                assert np.isnan(w[t]).all() == (t != 1)
                assert np.isnan(dx[t]).all() == (t != 1)
                assert not np.isnan(w[1]).any() and not np.isnan(dx[1]).any()


def test_nan_and_infinite_logits():
    x = np.array([[0.0, np.nan, 1.0, 0.5],
                  [np.inf, 0.0, 1.0, 0.5],
                  [-np.inf] * 4,
                  [-np.inf, 0.0, 1.0, 0.5]], dtype=np.float32)
    ind = np.array([[0, 2]] * 4)
    g = np.ones((4, 2))
    ws = selected_router_weights(x, ind, "softmax", False, 1.0, "f32")
    assert np.isnan(ws[:3]).all() and not np.isnan(ws[3]).any()
    assert ws[3, 0] == 0.0                 # exp(-inf) = 0, not poisoned
    dxs = selected_router_backward(x, ind, g, "softmax", False, 1.0, "f32")
    assert np.isnan(dxs[:3]).all() and not np.isnan(dxs[3]).any()
    wg = selected_router_weights(x, ind, "sigmoid", False, 1.0, "f32")
    assert not np.isnan(wg).any()          # the NaN logit is not selected
    assert wg[1].tolist() == [1.0, wg[0, 1]] and wg[2].tolist() == [0, 0]
    dxg = selected_router_backward(x, ind, g, "sigmoid", False, 1.0, "f32")
    assert dxg[0, 1] == 0.0 and dxg[1, 0] == 0.0 and dxg[2, 0] == 0.0
    assert not np.isnan(dxg).any()
    # renormalised sigmoid weights of two zero scores: 0/0
    wz = selected_router_weights(x[2:3], ind[:1], "sigmoid", True, 1.0, "f32")
    assert np.isnan(wz).all()


def test_option_limits():
    check_options(64, 64, "softmax", 1.0)
    check_options(3, 3, "sigmoid", 1e30)
    for E, k, sc, scale in ((8, 0, "softmax", 1.0), (8, 9, "softmax", 1.0),
                            (100, 65, "sigmoid", 1.0), (8, 2, "relu", 1.0),
                            (8, 2, "softmax", 0.0), (8, 2, "softmax", -1.0),
                            (8, 2, "softmax", math.inf),
                            (8, 2, "softmax", math.nan)):
        with pytest.raises(ValueError):
            check_options(E, k, sc, scale)


def test_gradient_rounds_to_the_logits_dtype():
    rng = np.random.default_rng(9)
    x, ind, g = _case(rng, 8, 16, 4)
    xb = torch.tensor(x).to(torch.bfloat16).float().numpy()
    d32 = selected_router_backward(xb, ind, g, "softmax", True, 1.0, "f32")
    db = selected_router_backward(xb, ind, g, "softmax", True, 1.0, "bf16")
    want = torch.tensor(d32).to(torch.bfloat16).double().numpy()
    # the float32 rounding first can differ from a direct bf16 rounding only
    # at exact ties, which random data does not hit
    assert np.array_equal(db, want)

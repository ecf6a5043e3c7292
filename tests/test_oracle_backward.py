"""Pins for the oracle's MoE backward chain (oracle.backward).

Contract: ruDNN user guide (RUDA docs, German edition), section 12; the
experts page's forward_dispatched_training and
ExpertTrainingCache::backward_with_strategy.
Pins, none of which reuses the oracle's own derivation:
* torch autograd in float64 through the whole layer written as a plain
  forward (fixed selection, FP32 routing weights as a leaf): every gradient
  of the chain (tokens, routing weights, gate, up, down weights);
* central finite differences of the layer's loss in float64;
* adjointness, exact on integer-valued data: dispatch backward is the
  transpose of dispatch, combine backward of combine;
* the training forward's expert outputs equal the inference forward's;
* the SwiGLU backward against autograd of SiLU(g) * u.
"""

import numpy as np
import pytest
import torch

from oracle.backward import (combine_backward, dispatch_backward,
                             experts_backward, experts_forward_training,
                             swiglu_backward)
from oracle.fp import round_to
from oracle.moe import combine, dispatch, experts


def _layer(rng, T, H, I, E, k, repeats=False):
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((E, I, H)) / np.sqrt(H)
    wu = rng.standard_normal((E, I, H)) / np.sqrt(H)
    wd = rng.standard_normal((E, H, I)) / np.sqrt(I)
    if repeats:
        idx = rng.integers(0, E, size=(T, k))
    else:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    w = rng.random((T, k)) + 0.1
    dout = rng.standard_normal((T, H))
    f32 = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
    return (f32(x), f32(wg), f32(wu), f32(wd), idx.astype(np.uint32), f32(w),
            f32(dout))


def _chain(x, wg, wu, wd, idx, w, dout, fmt):
    E = wg.shape[0]
    d = dispatch(x, idx, E)
    c = experts_forward_training(d["xd"], d["offsets"], wg, wu, wd, fmt)
    out = combine(c["y"], w, d["token_row"], fmt)
    dexp, dw = combine_backward(c["y"], w, d["token_row"], dout, fmt)
    b = experts_backward(d["xd"], d["offsets"], wg, wu, wd, c, dexp, fmt)
    dx = dispatch_backward(b["dinput"], d["token_row"], fmt)
    return dict(out=out, dx=dx, dw=dw, dgate=b["dgate"], dup=b["dup"],
                ddown=b["ddown"], d=d, c=c)


def _autograd(x, wg, wu, wd, idx, w, dout):
    t = lambda a: torch.tensor(a, dtype=torch.float64,  # noqa: E731
                               requires_grad=True)
    X, WG, WU, WD, W = t(x), t(wg), t(wu), t(wd), t(w)
    T, k = idx.shape
    out = []
    for i in range(T):
        acc = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(k):
            e = int(idx[i, j])
            g = WG[e] @ X[i]
            u = WU[e] @ X[i]
            a = torch.nn.functional.silu(g) * u
            acc = acc + W[i, j] * (WD[e] @ a)
        out.append(acc)
    out = torch.stack(out)
    (out * torch.tensor(dout)).sum().backward()
    return dict(out=out.detach().numpy(), dx=X.grad.numpy(),
                dw=W.grad.numpy(), dgate=WG.grad.numpy(),
                dup=WU.grad.numpy(), ddown=WD.grad.numpy())


@pytest.mark.parametrize("repeats", [False, True])
def test_chain_matches_autograd(repeats):
    rng = np.random.default_rng(3 + repeats)
    T, H, I, E, k = 9, 6, 10, 5, 3
    args = _layer(rng, T, H, I, E, k, repeats)
    got = _chain(*args, "f32")
    want = _autograd(*args)
    for key in ("out", "dx", "dw", "dgate", "dup", "ddown"):
        a, b = got[key], want[key]
        # float32 rounding at the page's rounding points, nothing else
        scale = np.abs(b).max()
        assert np.allclose(a, b, rtol=2e-6, atol=2e-6 * scale), key
    # experts no token selects get zero weight gradients
    used = np.zeros(E, dtype=bool)
    used[args[4].ravel()] = True
    for key in ("dgate", "dup", "ddown"):
        assert np.all(got[key][~used] == 0.0)


def test_chain_matches_finite_differences():
    rng = np.random.default_rng(11)
    T, H, I, E, k = 3, 3, 4, 3, 2
    x, wg, wu, wd, idx, w, dout = _layer(rng, T, H, I, E, k)
    got = _chain(x, wg, wu, wd, idx, w, dout, "f32")

    def loss(x_, wg_, wu_, wd_, w_):
        tot = 0.0
        for t in range(T):
            for j in range(k):
                e = int(idx[t, j])
                g = wg_[e] @ x_[t]
                u = wu_[e] @ x_[t]
                a = g * u / (1.0 + np.exp(-g))
                tot += w_[t, j] * float((wd_[e] @ a) @ dout[t])
        return tot

    params = [x, wg, wu, wd, w]
    names = ["dx", "dgate", "dup", "ddown", "dw"]
    h = 1e-6
    for p, name in enumerate(names):
        base = params[p]
        fd = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            hi = [q.copy() for q in params]
            lo = [q.copy() for q in params]
            hi[p][i] += h
            lo[p][i] -= h
            fd[i] = (loss(*hi) - loss(*lo)) / (2 * h)
        assert np.allclose(got[name], fd, rtol=1e-4,
                           atol=1e-5 * np.abs(fd).max()), name


def test_dispatch_backward_is_the_transpose_of_dispatch():
    rng = np.random.default_rng(5)
    T, H, E, k = 11, 4, 6, 3
    x = rng.integers(-8, 9, size=(T, H)).astype(np.float64)
    idx = rng.integers(0, E, size=(T, k)).astype(np.uint32)
    d = dispatch(x, idx, E)
    z = rng.integers(-8, 9, size=(T * k, H)).astype(np.float64)
    lhs = float((d["xd"] * z).sum())
    rhs = float((x * dispatch_backward(z, d["token_row"], "f32")).sum())
    assert lhs == rhs


def test_combine_backward_is_the_transpose_of_combine():
    rng = np.random.default_rng(6)
    T, H, E, k = 7, 5, 4, 2
    idx = rng.integers(0, E, size=(T, k)).astype(np.uint32)
    d = dispatch(np.zeros((T, H)), idx, E)
    y = rng.integers(-8, 9, size=(T * k, H)).astype(np.float64)
    w = rng.choice([0.25, 0.5, 1.0, 2.0], size=(T, k))
    dout = rng.integers(-8, 9, size=(T, H)).astype(np.float64)
    out = combine(y, w, d["token_row"], "f32")
    dexp, dw = combine_backward(y, w, d["token_row"], dout, "f32")
    assert float((out * dout).sum()) == float((y * dexp).sum())
    # d<out, dout>/dw[t,j] = dout[t] . y[row]
    for t in range(T):
        for j in range(k):
            assert dw[t, j] == float(dout[t] @ y[int(d["token_row"][t, j])])


def test_training_forward_equals_inference_forward():
    rng = np.random.default_rng(8)
    T, H, I, E, k = 20, 8, 12, 4, 2
    x, wg, wu, wd, idx, _, _ = _layer(rng, T, H, I, E, k)
    for fmt in ("f32", "bf16"):
        xr = round_to(x, fmt)
        wgr, wur, wdr = (round_to(a, fmt) for a in (wg, wu, wd))
        d = dispatch(xr, idx, E)
        c = experts_forward_training(d["xd"], d["offsets"], wgr, wur, wdr,
                                     fmt)
        y = experts(d["xd"], d["offsets"], wgr, wur, wdr, fmt)
        assert np.array_equal(c["y"], y)


def test_swiglu_backward_matches_autograd():
    rng = np.random.default_rng(9)
    g = rng.standard_normal(200) * 4
    u = rng.standard_normal(200)
    da = rng.standard_normal(200)
    dg, du = swiglu_backward(g, u, da, "f32")
    G = torch.tensor(g, requires_grad=True)
    U = torch.tensor(u, requires_grad=True)
    (torch.nn.functional.silu(G) * U * torch.tensor(da)).sum().backward()
    assert np.allclose(dg, G.grad.numpy(), rtol=1e-6, atol=1e-7)
    assert np.allclose(du, U.grad.numpy(), rtol=1e-6, atol=1e-7)


def test_rounding_points_in_bf16():
    """In bf16 every materialised tensor holds bf16 values and weight
    gradients hold FP32 values."""
    rng = np.random.default_rng(10)
    T, H, I, E, k = 6, 8, 8, 3, 2
    x, wg, wu, wd, idx, w, dout = (round_to(a, "bf16") if a.dtype.kind == "f"
                                   else a for a in _layer(rng, T, H, I, E, k))
    got = _chain(x, wg, wu, wd, idx, w, dout, "bf16")
    for key in ("dx",):
        assert np.array_equal(got[key], round_to(got[key], "bf16"))
    for key in ("gate", "up", "act", "y"):
        assert np.array_equal(got["c"][key], round_to(got["c"][key], "bf16"))
    for key in ("dw", "dgate", "dup", "ddown"):
        assert np.array_equal(got[key], round_to(got[key], "f32"))

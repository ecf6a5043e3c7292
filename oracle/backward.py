"""Plain CPU definition of the first-order MoE backward chain (test
infrastructure only; see the package docstring).

Sources: ruDNN user guide (RUDA docs, German edition), section 12
("first-order MoE training"), which orders the chain: combine backward gives
the expert-output gradient and FP32 weight gradients; the expert backward
gives the dispatched-row input gradient and FP32 gate, up and down weight
gradients; dispatch backward sums each token's selected rows without the
routing weights; the router backward turns the weight gradients into logits
gradients.  The experts page (docs.rs "ruDNN 0.1.25 source,
src/moe/experts.rs": forward_dispatched_training and
ExpertTrainingCache::backward_with_strategy) fixes what the training forward
keeps (the dispatched input, the raw gate and up products, the activation)
and the order of the expert backward: the down projection's backward, a
SwiGLU backward producing gate and up gradients, the gate and up
projections' backwards, and an elementwise add of their input gradients.

Readings where the pages leave a step open (also in the design notes):

* R-BPrec  every tensor the experts page materialises in the storage dtype
           is rounded to it once (gate_raw, up_raw, activated, the down
           backward's input gradient, the SwiGLU backward's two outputs, the
           gate and up backwards' input gradients, their sum); weight
           gradients are FP32 (rounded once from the exact value).  Every
           product is exact (float64 here) before its rounding.
* R-SwiB   SwiGLU backward of a = SiLU(g) * u with s = sigmoid(g):
           dg = da * u * s * (1 + g * (1 - s)), du = da * g * s.
* R-CombB  combine backward: the gradient of dispatched row r = (t, j) is
           w[t, j] * dout[t] (rounded to the dtype) and the weight gradient
           is the FP32 dot product dout[t] . y[r]; rows no slot maps to get
           no gradient (they do not exist in a complete dispatch).
* R-DispB  dispatch backward: dx[t] = sum over slots j of
           dinput[token_row[t, j]], in slot order, rounded once.
"""

import numpy as np

from .fp import decode, round_to
from .moe import silu_times


def _sigmoid(g):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def experts_forward_training(xd, offsets, w_gate, w_up, w_down, fmt):
    """Training forward over expert segments: returns dict gate, up, act, y
    ([N,I], [N,I], [N,I], [N,H]; float64 values of ``fmt``).  Rows past
    offsets[E] belong to no expert and stay zero."""
    xd = decode(xd, fmt)
    E = len(offsets) - 1
    N, H = xd.shape
    I = np.asarray(w_gate).shape[1]
    g = np.zeros((N, I))
    u = np.zeros((N, I))
    a = np.zeros((N, I))
    y = np.zeros((N, H))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        wg = decode(np.asarray(w_gate)[e], fmt)
        wu = decode(np.asarray(w_up)[e], fmt)
        wd = decode(np.asarray(w_down)[e], fmt)
        g[lo:hi] = round_to(xd[lo:hi] @ wg.T, fmt)
        u[lo:hi] = round_to(xd[lo:hi] @ wu.T, fmt)
        a[lo:hi] = round_to(silu_times(g[lo:hi], u[lo:hi]), fmt)
        y[lo:hi] = round_to(a[lo:hi] @ wd.T, fmt)
    return {"gate": g, "up": u, "act": a, "y": y}


def combine_backward(y, w, token_row, dout, fmt):
    """dexpert [N,H] (values of ``fmt``) and FP32 dweights [T,k] for the
    output gradient dout [T,H] of out[t] = sum_j w[t,j] * y[token_row[t,j]].
    w holds the routing weights as float64 values of their own format."""
    y = decode(y, fmt)
    dout = decode(dout, fmt)
    T, k = token_row.shape
    dexpert = np.zeros_like(y)
    dweights = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            r = int(token_row[t, j])
            dexpert[r] = round_to(w[t, j] * dout[t], fmt)
            dweights[t, j] = float(np.dot(dout[t], y[r]))
    return dexpert, round_to(dweights, "f32")


def swiglu_backward(g, u, da, fmt):
    """R-SwiB on stored (rounded) gate, up and activation-gradient values;
    both results rounded to ``fmt``."""
    s = _sigmoid(g)
    dg = round_to(da * u * s * (1.0 + g * (1.0 - s)), fmt)
    du = round_to(da * g * s, fmt)
    return dg, du


def _segments(offsets):
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo < hi:
            yield e, lo, hi


def down_backward(dy, act, offsets, w_down, fmt):
    """The down projection's backward: dact [N,I] = dy . w_down[e] (rounded
    to ``fmt``) and FP32 ddown [E,H,I] = dy_e^T . act_e."""
    dy = decode(dy, fmt)
    act = decode(act, fmt)
    E = len(offsets) - 1
    N, H = dy.shape
    I = act.shape[1]
    dact = np.zeros((N, I))
    ddown = np.zeros((E, H, I))
    for e, lo, hi in _segments(offsets):
        wd = decode(np.asarray(w_down)[e], fmt)
        dact[lo:hi] = round_to(dy[lo:hi] @ wd, fmt)
        ddown[e] = dy[lo:hi].T @ act[lo:hi]
    return dact, round_to(ddown, "f32")


def proj_backward(dz, xd, offsets, w, fmt):
    """The backward of z = xd . w[e]^T (gate or up): the input-gradient part
    dz . w[e] [N,H] (rounded to ``fmt``) and FP32 dw [E,I,H] = dz_e^T . xd_e."""
    dz = decode(dz, fmt)
    xd = decode(xd, fmt)
    E = len(offsets) - 1
    N, I = dz.shape
    H = xd.shape[1]
    dx = np.zeros((N, H))
    dw = np.zeros((E, I, H))
    for e, lo, hi in _segments(offsets):
        we = decode(np.asarray(w)[e], fmt)
        dx[lo:hi] = round_to(dz[lo:hi] @ we, fmt)
        dw[e] = dz[lo:hi].T @ xd[lo:hi]
    return dx, round_to(dw, "f32")


def experts_backward(xd, offsets, w_gate, w_up, w_down, cache, dy, fmt):
    """Expert backward from the training cache (gate, up, act) and the
    gradient dy [N,H] of the expert outputs.  Returns dict dinput [N,H]
    (values of ``fmt``) and FP32 dgate [E,I,H], dup [E,I,H], ddown [E,H,I],
    plus the intermediates dact, dg, du [N,I] and dxg, dxu [N,H], following
    the experts page's order and rounding points (R-BPrec)."""
    dact, ddown = down_backward(dy, cache["act"], offsets, w_down, fmt)
    dg, du = swiglu_backward(decode(cache["gate"], fmt),
                             decode(cache["up"], fmt), dact, fmt)
    dxg, dgate = proj_backward(dg, xd, offsets, w_gate, fmt)
    dxu, dup = proj_backward(du, xd, offsets, w_up, fmt)
    dinput = round_to(dxg + dxu, fmt)
    return {"dinput": dinput, "dgate": dgate, "dup": dup, "ddown": ddown,
            "dact": dact, "dg": dg, "du": du, "dxg": dxg, "dxu": dxu}


def dispatch_backward(dinput, token_row, fmt):
    """dx [T,H] = sum over slots of dinput[token_row[t, j]], one rounding."""
    dinput = decode(dinput, fmt)
    T, k = token_row.shape
    dx = np.zeros((T, dinput.shape[1]))
    for t in range(T):
        acc = np.zeros(dinput.shape[1])
        for j in range(k):
            acc = acc + dinput[int(token_row[t, j])]
        dx[t] = round_to(acc, fmt)
    return dx

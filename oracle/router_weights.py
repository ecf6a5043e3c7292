"""Plain CPU definition of router weights for a fixed selection and their
logits gradient (test infrastructure only; see the package docstring).

Source: ruDNN user guide (RUDA docs, German edition), section 12
("first-order MoE training"): ``selected_router_weights(logits, indices,
options)`` returns FP32 weights [T, top_k]; ``selected_router_backward(logits,
indices, grad_weights, options)`` returns the [T, E] logits gradient in the
logits dtype.  ``RouterWeightOptions`` picks softmax or sigmoid scoring,
optional renormalisation of the selected weights, then a finite positive
scale.  Indices are U32/I32/I64 with 1 <= top_k <= min(E, 64); a repeated
index gathers the same score again; an invalid index makes the whole row
NaN; only the continuous weights of the fixed selection are differentiated.

The weight of slot j of a row is, with u_j the score of expert i_j (softmax
over all E experts, or the sigmoid of the logit):

    w_j = scale * u_j                  without renormalisation
    w_j = scale * u_j / sum_l u_l      with renormalisation

and the gradient is the exact vector-Jacobian product
dL/dx_e = sum_j g_j * dw_j/dx_e for grad_weights g.  Worked out:

    a_j = scale * g_j                                      (no renorm)
    a_j = (scale / S) * (g_j - sum_l g_l u_l / S)          (renorm, S = sum u)
    A_e = sum over slots j with i_j == e of a_j            (gather: repeats add)
    softmax:  dL/dx_e = p_e * (A_e - sum_j u_j a_j)
    sigmoid:  dL/dx_e = s_e * (1 - s_e) * A_e   if e is selected, else 0

Readings where the section leaves a step open (also in the design notes):

* R-WPrec  both results are computed exactly (float64 here) and rounded
           once: weights to FP32, the gradient to the logits dtype.  The
           section fixes the output types only.
* R-WNaN   scores are evaluated as defined, so NaN propagates the way the
           arithmetic carries it: under softmax a row holding a NaN, a +inf
           or only -inf has NaN scores everywhere (the max subtraction
           gives inf - inf or a NaN); under sigmoid only the scores of NaN
           logits are NaN (sigmoid(+-inf) = 1, 0).
* R-WInv   an index is invalid if it is negative (signed types) or >= E;
           one invalid index makes the row's weights and its whole
           gradient row NaN.
* R-WZero  under sigmoid scoring a logit that no slot selects does not
           enter the weights, so its gradient is exactly 0 (even when the
           logit is NaN or infinite); under softmax every logit enters
           through the normaliser.
"""

import math

import numpy as np

from .fp import decode, round_to

SCORINGS = ("softmax", "sigmoid")


def check_options(E, k, scoring, scale):
    """The limits of the guide's section 12 (ValueError when violated)."""
    if scoring not in SCORINGS:
        raise ValueError("scoring must be softmax or sigmoid")
    if not 1 <= k <= min(E, 64):
        raise ValueError("top_k must satisfy 1 <= top_k <= min(E, 64)")
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and positive")


def scores(row, scoring):
    """float64 scores of one row of logits (softmax over the row, or the
    sigmoid of each logit), NaN propagating as the arithmetic does."""
    row = np.asarray(row, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        if scoring == "softmax":
            q = np.exp(row - row.max())
            return q / q.sum()
        return 1.0 / (1.0 + np.exp(-row))


def _row_valid(ind, E):
    return all(0 <= int(i) < E for i in ind)


def _slot_terms(u, g, renormalize, scale):
    """a_j of the gradient (see the module docstring)."""
    if not renormalize:
        return scale * g
    S = u.sum()
    return (scale / S) * (g - (g * u).sum() / S)


def selected_router_weights(logits, indices, scoring, renormalize, scale,
                            fmt):
    """logits [T,E] values of ``fmt``; indices [T,k] integers (any numpy
    integer type; values as stored).  Returns float64 [T,k] holding FP32
    values."""
    lg = decode(logits, fmt)
    T, E = lg.shape
    ind = np.asarray(indices).astype(np.int64)
    k = ind.shape[1]
    check_options(E, k, scoring, scale)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        if not _row_valid(ind[t], E):
            w[t] = np.nan
            continue
        u = scores(lg[t], scoring)[ind[t]]
        with np.errstate(invalid="ignore", divide="ignore"):
            w[t] = scale * (u / u.sum() if renormalize else u)
    return round_to(w, "f32")


def selected_router_backward(logits, indices, grad_weights, scoring,
                             renormalize, scale, fmt):
    """The [T,E] logits gradient for FP32 grad_weights [T,k], rounded to
    ``fmt`` (float64 values)."""
    lg = decode(logits, fmt)
    T, E = lg.shape
    ind = np.asarray(indices).astype(np.int64)
    k = ind.shape[1]
    check_options(E, k, scoring, scale)
    gw = np.asarray(grad_weights, dtype=np.float64)
    dx = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        if not _row_valid(ind[t], E):
            dx[t] = np.nan
            continue
        p = scores(lg[t], scoring)
        u = p[ind[t]]
        with np.errstate(invalid="ignore", divide="ignore"):
            a = _slot_terms(u, gw[t], renormalize, scale)
            A = np.zeros(E)
            for j in range(k):
                A[ind[t, j]] += a[j]
            if scoring == "softmax":
                dx[t] = p * (A - (u * a).sum())
            else:
                sel = np.zeros(E, dtype=bool)
                sel[ind[t]] = True
                dx[t] = np.where(sel, p * (1.0 - p) * A, 0.0)
    return round_to(dx, fmt)

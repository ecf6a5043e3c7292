"""Plain CPU definition of group-limited sigmoid routing (test infrastructure
only; see the package docstring).

Source: ruDNN user guide (RUDA docs, German edition), section 10
("group-limited sigmoid MoE routing"): ``route_sigmoid_grouped(logits, bias,
options)`` and ``GroupRoutingOptions`` (top_k, groups, selected_groups,
group_top_two, renormalize, scale); the experts page (docs.rs "ruDNN 0.1.25
source, src/moe/experts.rs", ``forward_sigmoid_grouped``) chains it with the
same dispatch, experts and combine as the softmax path.

What the section fixes: logits [T,E] in F32/F16/BF16; an optional FP32
correction bias [E] that changes only the selection; experts split into
``groups`` equal groups of consecutive ids; a group's score is its largest
corrected value, or with ``group_top_two`` the sum of its two largest; the
``selected_groups`` best groups are kept, then the top_k experts among them;
the weights are the original (uncorrected) sigmoid values, optionally
renormalised, then multiplied by ``scale``; ties go to the smaller id.
Limits: 1 <= E <= 1024, 1 <= groups <= 128 dividing E, 1 <= top_k <= 64,
top_k <= selected_groups * E / groups, at least two experts per group with
group_top_two, scale finite and positive.

Readings where the section leaves a step open (also listed, with reasons, in
the repository's design notes):

* R-Sig     the FP32 sigmoid of a logit is the float64 value of
            1 / (1 + exp(-x)) rounded once to float32 (round to nearest
            even): the correctly rounded FP32 sigmoid up to events of
            probability ~1e-9, so the selection, which compares computed
            FP32 values, is the same wherever it is evaluated.
* R-Corr    corrected value c_e = FP32(sigmoid_e + bias_e) (bias 0 when
            absent); group scores are FP32 (max, or the FP32 sum of the two
            largest).
* R-GTie    groups tie by score to the smaller group id, like experts.
* R-SOrder  the k slots are in selection order: corrected value descending,
            then id ascending.
* R-SNaN    a row whose corrected values or group scores hold a NaN (a NaN
            logit or bias entry, or +inf and -inf bias values summed in one
            group) has no order: indices 0..k-1 and NaN weights, as for the
            softmax path.
* R-SCast   weights are computed in FP32 (renormalising denominator: the
            FP32 sum of the selected sigmoid values in slot order), then
            multiplied by the FP32 scale, then rounded to the logits dtype.
            When every chosen sigmoid value is 0 the renormalised weights
            are 0/0 = NaN, the plain result of the definition.
"""

import math

import numpy as np

from .fp import decode, round_to
from .moe import combine, dispatch, expert_rows, experts


def check_options(E, k, groups, selected_groups, group_top_two, scale):
    """The limits of the guide's section 10 (ValueError when violated)."""
    if not 1 <= E <= 1024:
        raise ValueError("expert count must be in 1..=1024")
    if not 1 <= groups <= 128 or E % groups:
        raise ValueError("groups must be in 1..=128 and divide the experts")
    if not 1 <= selected_groups <= groups:
        raise ValueError("selected_groups must be in 1..=groups")
    if not 1 <= k <= 64 or k > selected_groups * (E // groups):
        raise ValueError("top_k must be in 1..=64 and fit the selected groups")
    if group_top_two and E // groups < 2:
        raise ValueError("group_top_two needs two experts per group")
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and positive")


def sigmoid_fp32(x):
    """R-Sig: float64 evaluation of 1/(1+exp(-x)), one rounding to float32."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def group_scores(c, groups, group_top_two):
    """R-Corr: per group of consecutive experts, the largest corrected value
    or the FP32 sum of the two largest."""
    size = len(c) // groups
    out = np.zeros(groups, dtype=np.float32)
    for g in range(groups):
        vals = sorted((float(v) for v in c[g * size:(g + 1) * size]),
                      reverse=True)
        if group_top_two:
            with np.errstate(invalid="ignore"):          # inf + -inf: NaN
                out[g] = np.float32(np.float32(vals[0]) + np.float32(vals[1]))
        else:
            out[g] = np.float32(vals[0])
    return out


def route_sigmoid_grouped(logits, bias, k, groups, selected_groups,
                          group_top_two, renormalize, scale, fmt):
    """Route one batch (guide section 10).

    logits: [T,E] values of ``fmt``; bias: None or [E] float32 values.
    Returns (idx uint32 [T,k], w float64 [T,k] holding ``fmt`` values).
    """
    lg = decode(logits, fmt).astype(np.float32)      # exact upcast
    T, E = lg.shape
    check_options(E, k, groups, selected_groups, group_top_two, scale)
    b = (np.zeros(E, dtype=np.float32) if bias is None
         else np.asarray(bias, dtype=np.float32))
    size = E // groups
    sc = np.float32(scale)
    idx = np.zeros((T, k), dtype=np.uint32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        s = sigmoid_fp32(lg[t])
        c = (s + b).astype(np.float32)
        gs = group_scores(c, groups, group_top_two)
        if np.isnan(c).any() or np.isnan(gs).any():     # R-SNaN
            idx[t] = np.arange(k)
            w[t] = np.nan
            continue
        best_groups = sorted(range(groups),
                             key=lambda g: (-float(gs[g]), g))[:selected_groups]
        eligible = [e for e in range(E) if e // size in best_groups]
        sel = sorted(eligible, key=lambda e: (-float(c[e]), e))[:k]
        ws = s[sel].astype(np.float32)
        if renormalize:
            den = np.float32(0.0)
            for v in ws:
                den = np.float32(den + v)
            with np.errstate(invalid="ignore"):      # 0/0 stays NaN
                ws = (ws / den).astype(np.float32)
        ws = (ws * sc).astype(np.float32)
        idx[t] = sel
        w[t] = round_to(ws.astype(np.float64), fmt)
    return idx, w


def forward_sigmoid_grouped(x, logits, bias, w_gate, w_up, w_down, k, groups,
                            selected_groups, group_top_two, renormalize,
                            scale, fmt, logits_fmt=None):
    """route_sigmoid_grouped -> dispatch -> experts -> combine (experts page,
    forward_sigmoid_grouped).  Returns a dict of every stage's result."""
    lfmt = fmt if logits_fmt is None else logits_fmt
    E = np.asarray(w_gate).shape[0]
    idx, w = route_sigmoid_grouped(logits, bias, k, groups, selected_groups,
                                   group_top_two, renormalize, scale, lfmt)
    d = dispatch(decode(x, fmt), idx, E)
    y = experts(d["xd"], d["offsets"], w_gate, w_up, w_down, fmt)
    out = combine(y, w, d["token_row"], fmt)
    return {"idx": idx, "w": w, "dispatch": d, "y": y, "out": out}


def forward_sigmoid_tokens(x, logits, bias, w_gate, w_up, w_down, k, groups,
                           selected_groups, group_top_two, renormalize,
                           scale, fmt, tokens, logits_fmt=None):
    """The forward output for selected tokens only, computed token by token
    (route the token's logits, apply its k experts to its row, combine), for
    sizes where the full forward is too slow for the oracle."""
    lfmt = fmt if logits_fmt is None else logits_fmt
    x64 = decode(x, fmt)
    idx, w = route_sigmoid_grouped(np.asarray(logits)[list(tokens)], bias, k,
                                   groups, selected_groups, group_top_two,
                                   renormalize, scale, lfmt)
    out = np.zeros((len(tokens), x64.shape[1]), dtype=np.float64)
    for n, t in enumerate(tokens):
        acc = np.zeros(x64.shape[1], dtype=np.float64)
        for j in range(k):
            e = int(idx[n, j])
            y = expert_rows(x64[t][None, :], e,
                            decode(np.asarray(w_gate)[e], fmt),
                            decode(np.asarray(w_up)[e], fmt),
                            decode(np.asarray(w_down)[e], fmt), fmt)[0]
            acc = acc + w[n, j] * y
        out[n] = round_to(acc, fmt)
    return idx, w, out

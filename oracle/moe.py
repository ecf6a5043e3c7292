"""Plain CPU definition of the local MoE forward pass (test infrastructure only).

Sources (cited by page title and section):

* [Guide] ruDNN user guide (RUDA docs, German edition):
  section 3 "MoE workflow", section 4 "routing contract",
  section 5 "expert weights and dispatch", section 6 "calling MoE".
* [Experts] docs.rs "ruDNN 0.1.25 source, src/moe/experts.rs":
  ``SwiGluExperts::new`` and ``forward_dispatched_with_strategy``.

Pipeline ([Guide] section 3): logits -> softmax/top-k -> compact dispatch ->
SwiGLU experts -> weighted combine.

Readings taken where the pages leave a step open (each is also listed with
its reason in the design notes of the repository):

* R-Key   top-k ranks experts by the FP32 logit, descending, then by expert
          id, ascending.  The softmax is strictly increasing in the logit, so
          this is exactly "top-k of the softmax" with the guide's tie rule.
* R-Order the k slots of a row are in that same order (best first).
* R-NaN   a poisoned row (any NaN, any +inf, or every entry -inf) gets
          indices 0..k-1 (every expert ties, ties go to lower ids) and NaN
          weights.
* R-Cast  weights are cast to the logits dtype with round-to-nearest-even in
          both modes (renormalised or not).
* R-Renorm the renormalising denominator is the FP32 sum of the selected
          probabilities in slot order.
* R-Disp  dispatch is stable: row-major (token, slot) order inside each
          expert segment.  The guide leaves the in-expert order open, so
          tests compare per-expert token multisets plus everything that is
          unique (counts, offsets, segment of each row).
* R-Prec  gate, up, act and the expert output are rounded to the weight
          dtype where the experts page materialises them as tensors; the
          products themselves are exact sums (float64) rounded once.
* R-SwiGLU act = SiLU(gate) * up, SiLU(g) = g / (1 + exp(-g)); no clamp and
          no alpha.
* R-Clip  the clipped variant (MindSpeed-Ops page, ``clipped_swiglu``
          parameter table: swiglu_alpha, default 1.702, and swiglu_limit L
          >= 0, default 7, with the gate clamped from above at L and up to
          [-L, L]; the page shows no formula): act = gc * sigmoid(alpha * gc)
          * uc with gc = min(gate, L), uc = min(max(up, -L), L), the plain
          swish-with-parameter reading of "SwiGLU's alpha".  NaN propagates
          through the clamps.
* R-Comb  combine sums w[t,j] * y[t,j] over the k slots and rounds once to
          the activation dtype; the routing weights are applied here only.
"""

import numpy as np

from .fp import decode, round_to


# ---------------------------------------------------------------------------
# Routing ([Guide] section 4)
# ---------------------------------------------------------------------------

def is_poisoned(row):
    """[Guide] section 4: a row holding NaN, +inf, or only -inf keeps NaN
    weights instead of falling back to a uniform distribution."""
    return bool(np.isnan(row).any() or (row == np.inf).any()
                or (row == -np.inf).all())


def softmax_fp32(row):
    """[Guide] section 4: the softmax over all E experts is taken in FP32
    before top-k.  ``row`` holds float32 logits with a finite maximum.
    Returns float32 probabilities (sum taken left to right)."""
    row = row.astype(np.float32)
    m = np.float32(row.max())
    q = np.exp(row - m).astype(np.float32)
    s = np.float32(0.0)
    for v in q:
        s = np.float32(s + v)
    return (q / s).astype(np.float32)


def rank_experts(row):
    """R-Key: expert ids ordered by (logit descending, id ascending)."""
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))


def route(logits, k, renormalize, fmt):
    """Route one batch.

    logits: [T,E] values of ``fmt`` (any numpy form ``decode`` accepts).
    Returns (idx uint32 [T,k], w float64 [T,k] holding ``fmt`` values).
    """
    lg = decode(logits, fmt).astype(np.float32)      # exact upcast
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("top_k must satisfy 1 <= top_k <= E")
    idx = np.zeros((T, k), dtype=np.uint32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        row = lg[t]
        if is_poisoned(row):
            idx[t] = np.arange(k)
            w[t] = np.nan
            continue
        p = softmax_fp32(row)
        sel = rank_experts(row)[:k]
        ps = p[sel]
        if renormalize:
            den = np.float32(0.0)
            for v in ps:
                den = np.float32(den + v)
            ps = (ps / den).astype(np.float32)
        idx[t] = sel
        w[t] = round_to(ps.astype(np.float64), fmt)
    return idx, w


# ---------------------------------------------------------------------------
# Dispatch ([Guide] section 5; [Experts] forward_dispatched_with_strategy)
# ---------------------------------------------------------------------------

def dispatch(x, idx, E):
    """Compact, expert-contiguous dispatch with no capacity drop.

    x:   [T,H] token rows (any dtype; rows are copied bit for bit)
    idx: [T,k] expert of each (token, slot)
    Returns a dict with
      counts     [E]   rows per expert
      offsets    [E+1] segment starts, offsets[E] == T*k
      row_expert [N]   expert of each dispatched row
      row_token  [N]   source token of each dispatched row
      token_row  [T,k] dispatched row of each (token, slot)  (the stored
                       mapping that restores token order)
      xd         [N,H] dispatched rows
    """
    T, k = idx.shape
    N = T * k
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            counts[int(idx[t, j])] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = np.zeros(E, dtype=np.int64)
    row_expert = np.zeros(N, dtype=np.uint32)
    row_token = np.zeros(N, dtype=np.uint32)
    token_row = np.zeros((T, k), dtype=np.uint32)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            r = offsets[e] + cursor[e]
            cursor[e] += 1
            row_expert[r] = e
            row_token[r] = t
            token_row[t, j] = r
    xd = np.asarray(x)[row_token]
    return {"counts": counts, "offsets": offsets, "row_expert": row_expert,
            "row_token": row_token, "token_row": token_row, "xd": xd}


# ---------------------------------------------------------------------------
# SwiGLU experts ([Experts] forward_dispatched_with_strategy)
# ---------------------------------------------------------------------------

def silu_times(g, u):
    """R-SwiGLU: SiLU(g) * u = g * u / (1 + exp(-g)), in float64."""
    with np.errstate(over="ignore"):
        return g * u / (1.0 + np.exp(-g))


def clipped_silu_times(g, u, alpha, limit):
    """R-Clip, the clipped SwiGLU of the MindSpeed-Ops page (``clipped_swiglu``
    parameter table): the gate is clamped from above at ``limit``, the up
    value to [-limit, limit], and the activation is the swish with parameter
    ``alpha`` of the clamped gate times the clamped up value:
    gc * u_c / (1 + exp(-alpha * gc)), float64, NaN propagating."""
    gc = np.minimum(g, limit)
    uc = np.minimum(np.maximum(u, -limit), limit)
    with np.errstate(over="ignore"):
        return gc * uc / (1.0 + np.exp(-alpha * gc))


def expert_rows(xd, e, w_gate, w_up, w_down, fmt, clip=None):
    """One expert applied to rows ``xd`` [n,H] (float64 values of ``fmt``).

    gate/up: [I,H] slices of the [E,I,H] weights; down: [H,I] slice of the
    [E,H,I] weight ([Experts] ``SwiGluExperts::new`` doc comment).  Each
    product is an exact float64 matrix product rounded once; gate, up and act
    are rounded to ``fmt`` as the experts page stores them (R-Prec).
    """
    return expert_down(expert_act(xd, w_gate, w_up, fmt, clip), w_down, fmt)


def expert_down(act, w_down, fmt):
    """The down product of one expert's activation rows: act [n,I] times the
    transpose of its [H,I] down weight, an exact float64 sum rounded once to
    ``fmt`` (R-Prec).  Output columns are independent, so a slice of the
    weight's rows gives the matching slice of the columns."""
    return round_to(act @ w_down.T, fmt)


def expert_act(xd, w_gate, w_up, fmt, clip=None):
    """The activation rows of one expert, act = SwiGLU(gate, up) [n,I]: the
    gate and up products (exact float64 sums rounded once to ``fmt``), then
    SiLU(gate) * up (or the clipped form) rounded to ``fmt`` ([Experts]
    forward_dispatched_with_strategy stores gate, up and this result as
    tensors of the weight dtype; R-Prec)."""
    g = round_to(xd @ w_gate.T, fmt)
    u = round_to(xd @ w_up.T, fmt)
    return round_to(silu_times(g, u) if clip is None
                    else clipped_silu_times(g, u, *clip), fmt)


def experts(xd, offsets, w_gate, w_up, w_down, fmt, rows=None, clip=None,
            with_act=False):
    """Grouped SwiGLU over expert segments.

    xd [N,H], offsets [E+1]; weights in ``fmt`` (decoded here).  If ``rows``
    is given, only those dispatched rows are computed (returned in that
    order); otherwise all N rows.  ``clip`` = (alpha, limit) selects the
    clipped SwiGLU activation.  With ``with_act`` the activation rows
    [len(rows), I] are returned too, as (y, act); rows of no expert give
    zeros in both.
    """
    xd = decode(xd, fmt)
    E = len(offsets) - 1
    N, H = xd.shape
    I = np.asarray(w_gate).shape[1]
    want = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(want), H), dtype=np.float64)
    act = np.zeros((len(want), I), dtype=np.float64)
    seg = np.searchsorted(np.asarray(offsets), want, side="right") - 1
    for e in range(E):
        sel = np.nonzero(seg == e)[0]
        if len(sel) == 0:
            continue
        wg = decode(np.asarray(w_gate)[e], fmt)
        wu = decode(np.asarray(w_up)[e], fmt)
        wd = decode(np.asarray(w_down)[e], fmt)
        assert wg.shape == (I, H) and wd.shape == (H, I)
        a = expert_act(xd[want[sel]], wg, wu, fmt, clip)
        act[sel] = a
        out[sel] = expert_down(a, wd, fmt)
    return (out, act) if with_act else out


# ---------------------------------------------------------------------------
# Combine ([Guide] section 6; weights applied here only)
# ---------------------------------------------------------------------------

def combine(y, w, token_row, fmt, tokens=None):
    """out[t] = round(sum_j w[t,j] * y[token_row[t,j]]), float64 sum.

    y [N,H] expert outputs (values of ``fmt``), w [T,k] routing weights
    (float64 values), token_row [T,k].  ``tokens`` restricts the output to
    those token ids.
    """
    T, k = token_row.shape
    want = range(T) if tokens is None else tokens
    y = decode(y, fmt)
    out = []
    for t in want:
        acc = np.zeros(y.shape[1], dtype=np.float64)
        for j in range(k):
            acc = acc + w[t, j] * y[int(token_row[t, j])]
        out.append(round_to(acc, fmt))
    return np.array(out).reshape(len(out), y.shape[1])


# ---------------------------------------------------------------------------
# Whole forward ([Experts] SwiGluExperts::forward)
# ---------------------------------------------------------------------------

def forward(x, logits, w_gate, w_up, w_down, k, renormalize, fmt,
            logits_fmt=None):
    """route -> dispatch -> experts -> combine.  Returns a dict of every
    stage's result (float64 values of the storage formats)."""
    lfmt = fmt if logits_fmt is None else logits_fmt
    E = np.asarray(w_gate).shape[0]
    idx, w = route(logits, k, renormalize, lfmt)
    d = dispatch(decode(x, fmt), idx, E)
    y = experts(d["xd"], d["offsets"], w_gate, w_up, w_down, fmt)
    out = combine(y, w, d["token_row"], fmt)
    return {"idx": idx, "w": w, "dispatch": d, "y": y, "out": out}


def forward_tokens(x, logits, w_gate, w_up, w_down, k, renormalize, fmt,
                   tokens, logits_fmt=None):
    """The forward output for selected tokens only, computed token by token:
    route the token's logits, apply its k experts to its row, combine.
    Used at sizes where the full forward is too slow for the oracle."""
    lfmt = fmt if logits_fmt is None else logits_fmt
    x64 = decode(x, fmt)
    idx, w = route(np.asarray(logits)[list(tokens)], k, renormalize, lfmt)
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

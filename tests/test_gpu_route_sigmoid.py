"""GPU parity of group-limited sigmoid routing (ruDNN user guide, section
10) and of the forward built on it (experts page, forward_sigmoid_grouped)
against the oracle.  Indices bit exact; weights and outputs within the
tolerances of parity_util; poisoned rows identical."""

import json
import os

import numpy as np
import pytest
import torch

import mixture_experts_layer_28_amd as moe
from mixture_experts_layer_28_amd import workloads
from oracle.grouped import (forward_sigmoid_grouped, forward_sigmoid_tokens,
                            route_sigmoid_grouped)
from parity_util import assert_close, u32, values

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "sigmoid_grouped_cases.json")
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
FMT = {v: k for k, v in TDT.items()}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(lg_t, bias, k, groups, sg, top_two, renorm, scale, what):
    """Route on the GPU and with the oracle; compare; return oracle idx."""
    fmt = FMT[lg_t.dtype]
    b_t = None if bias is None else torch.from_numpy(bias).cuda()
    print("case:", what, flush=True)
    idx_g, w_g = moe.moe_route_sigmoid_grouped(
        lg_t.cuda(), k, groups, sg, bias=b_t, group_top_two=top_two,
        renormalize=renorm, scale=scale)
    torch.cuda.synchronize()
    idx_r, w_r = route_sigmoid_grouped(values(lg_t), bias, k, groups, sg,
                                       top_two, renorm, scale, fmt)
    np.testing.assert_array_equal(u32(idx_g), idx_r, err_msg=what)
    assert_close(values(w_g), w_r, fmt, what)
    return idx_r


def _val(v):
    return {"nan": np.nan, "inf": np.inf, "-inf": -np.inf}.get(v, v)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_golden_cases(fmt):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if "logits" in c:
            row = np.array([[_val(v) for v in c["logits"]]], dtype=np.float32)
        else:
            p = np.array(c["p"], dtype=np.float64)
            row = np.log(p / (1.0 - p)).astype(np.float32)[None, :]
        lg = torch.from_numpy(row).to(TDT[fmt])
        bias = (None if "bias" not in c else
                np.array([_val(v) for v in c["bias"]], dtype=np.float32))
        idx = _check(lg, bias, c["k"], c["groups"], c["selected_groups"],
                     c["group_top_two"], c["renormalize"], c["scale"],
                     "%s %s" % (c["name"], fmt))
        if fmt == "f32":
            assert idx[0].tolist() == c["idx"], c["name"]


# (E, groups, selected_groups, top_two, k): every lanes-per-row split of the
# kernel (E <= 8 ... E <= 1024), groups smaller and larger than the lanes of
# a row, one group, groups of one expert, k up to 64 and up to the kept
# experts
CONFIGS = [
    (1, 1, 1, False, 1), (2, 1, 1, True, 2), (3, 3, 2, False, 2),
    (6, 2, 1, True, 3), (8, 4, 2, True, 4), (8, 8, 3, False, 3),
    (12, 3, 2, True, 5), (16, 16, 5, False, 5), (24, 4, 2, True, 12),
    (32, 8, 3, True, 6), (40, 5, 2, False, 16), (64, 8, 4, True, 8),
    (64, 1, 1, False, 64), (64, 64, 8, False, 8), (96, 12, 5, True, 10),
    (128, 16, 4, True, 8), (160, 10, 3, False, 20), (256, 8, 4, True, 8),
    (256, 128, 16, True, 32), (384, 3, 1, True, 64), (512, 64, 8, False, 16),
    (600, 120, 30, True, 64), (1024, 128, 16, True, 64), (1024, 1, 1, True, 8),
    (1024, 16, 3, False, 40),
]


@pytest.mark.parametrize("E,groups,sg,top_two,k", CONFIGS)
def test_random_configs(E, groups, sg, top_two, k):
    rng = np.random.default_rng(E * 1000 + groups)
    T = 300
    # a coarse grid forces equal scores (experts and groups), a little noise
    # on odd E separates them
    lg = (rng.integers(-6, 7, size=(T, E)) * 0.5
          + rng.standard_normal((T, E)) * 0.01 * (E % 2)).astype(np.float32)
    bias = (rng.integers(-2, 3, size=E) * 0.125).astype(np.float32)
    fmts = ("f32", "bf16") if E <= 256 else ("bf16",)
    for fmt in fmts:
        for b, renorm, scale in ((None, True, 1.0), (bias, False, 2.5),
                                 (bias, True, 0.75)):
            _check(torch.from_numpy(lg).to(TDT[fmt]), b, k, groups, sg,
                   top_two, renorm, scale,
                   "E=%d g=%d sg=%d t2=%d k=%d %s bias=%s r=%d" % (
                       E, groups, sg, top_two, k, fmt, b is not None,
                       renorm))


def test_special_values():
    rng = np.random.default_rng(3)
    T, E = 257, 16
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[3, 5] = np.nan              # poisoned row
    lg[9, 0] = np.inf              # sigmoid 1, an ordinary score
    lg[10] = -np.inf               # every score 0: ties everywhere
    lg[11, ::2] = -np.inf
    lg[12, 7] = -0.0
    lg[13] = 120.0                 # sigmoid rounds to 1 for all
    lg[14] = -120.0                # sigmoid underflows to 0
    lg[15, :4] = -100.0            # subnormal sigmoid values
    lg[15, 4:6] = -103.0           # the smallest subnormal
    for fmt in ("f32", "f16", "bf16"):
        for top_two in (False, True):
            for renorm in (False, True):
                _check(torch.from_numpy(lg).to(TDT[fmt]), None, 4, 4, 2,
                       top_two, renorm, 1.0,
                       "special %s t2=%d r=%d" % (fmt, top_two, renorm))
    # infinite bias entries: a -inf entry is never chosen while others can
    # be; +inf and -inf summed in one group poison every row
    bias = np.zeros(E, dtype=np.float32)
    bias[1] = -np.inf
    bias[6] = np.inf
    _check(torch.from_numpy(lg), bias, 4, 4, 2, True, True, 1.0, "inf bias")
    bias[7] = -np.inf
    bias[4:6] = -np.inf
    idx = _check(torch.from_numpy(lg), bias, 4, 8, 2, True, True, 1.0,
                 "inf bias poisons")
    assert (idx == np.arange(4)).all()
    bias[:] = 0
    bias[2] = np.nan               # a NaN bias entry poisons every row
    _check(torch.from_numpy(lg), bias, 4, 4, 2, False, True, 1.0, "nan bias")


def test_empty_batch():
    lg = torch.zeros((0, 64), device="cuda", dtype=torch.bfloat16)
    idx, w = moe.moe_route_sigmoid_grouped(lg, 8, 8, 4)
    assert idx.shape == (0, 8) and w.shape == (0, 8)


def test_full_size_workload():
    """The grouped workload's routing at full size (T=8192, E=64)."""
    wl = workloads.make("grouped", H=8, I=8)
    idx = _check(wl["logits"], wl["bias"].numpy(), wl["k"], wl["groups"],
                 wl["selected_groups"], wl["group_top_two"], wl["renorm"],
                 wl["scale"], "grouped T=8192")
    # every row's experts come from at most selected_groups groups
    g = idx.astype(np.int64) // (wl["E"] // wl["groups"])
    assert max(len(set(r)) for r in g.tolist()) <= wl["selected_groups"]


def test_many_rows_wrap_the_grid():
    """More rows than one pass of the capped grid covers (65536 blocks of 4
    rows at E=1024): rows on both sides of the wrap, sampled."""
    E, groups, sg, k = 1024, 32, 8, 16
    T = 65536 * 4 + 37
    gen = torch.Generator(device="cuda").manual_seed(5)
    lg = torch.randn((T, E), generator=gen, device="cuda").to(torch.bfloat16)
    print("case: T=%d E=%d" % (T, E), flush=True)
    idx_g, w_g = moe.moe_route_sigmoid_grouped(lg, k, groups, sg,
                                               group_top_two=True)
    torch.cuda.synchronize()
    rows = [0, 1, 262143, 262144, 262145, T - 1] + list(
        np.random.default_rng(0).choice(T, size=10, replace=False))
    sel = torch.tensor(rows, device="cuda")
    idx_r, w_r = route_sigmoid_grouped(values(lg[sel]), None, k, groups, sg,
                                       True, True, 1.0, "bf16")
    np.testing.assert_array_equal(u32(idx_g[sel]), idx_r)
    assert_close(values(w_g[sel]), w_r, "bf16", "wrap")


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def _np(wl, key):
    return workloads.to_numpy(wl[key], wl["fmt"])


@pytest.mark.parametrize("T,H,I,E,k,groups,sg,top_two", [
    (45, 136, 200, 8, 2, 4, 2, True), (260, 64, 96, 12, 3, 3, 2, False),
    (1, 32, 16, 4, 4, 2, 2, True), (300, 32, 24, 256, 8, 8, 4, True)])
def test_forward_small(T, H, I, E, k, groups, sg, top_two):
    wl = workloads.make("edge", T=T, H=H, I=I, E=E, k=k)
    for name in ("x", "logits", "w_gate", "w_up", "w_down"):
        wl[name] = wl[name].to(torch.bfloat16)
    wl["fmt"] = "bf16"
    bias = (np.random.default_rng(T).standard_normal(E) * 0.25).astype(
        np.float32)
    c = {key: wl[key].cuda() for key in ("x", "logits", "w_gate", "w_up",
                                          "w_down")}
    print("case: forward T=%d E=%d" % (T, E), flush=True)
    out = moe.moe_forward_sigmoid_grouped(
        c["x"], c["logits"], c["w_gate"], c["w_up"], c["w_down"], k, groups,
        sg, bias=torch.from_numpy(bias).cuda(), group_top_two=top_two,
        renormalize=True, scale=2.5)
    torch.cuda.synchronize()
    ref = forward_sigmoid_grouped(_np(wl, "x"), _np(wl, "logits"), bias,
                                  _np(wl, "w_gate"), _np(wl, "w_up"),
                                  _np(wl, "w_down"), k, groups, sg, top_two,
                                  True, 2.5, "bf16")
    assert_close(values(out), ref["out"], "bf16", "forward")


def test_staged_equals_one_call():
    wl = workloads.make("grouped", T=300, H=128, I=192, device="cuda")
    args = (wl["k"], wl["groups"], wl["selected_groups"])
    opts = dict(bias=wl["bias"], group_top_two=wl["group_top_two"],
                renormalize=wl["renorm"], scale=wl["scale"])
    one = moe.moe_forward_sigmoid_grouped(wl["x"], wl["logits"], wl["w_gate"],
                                          wl["w_up"], wl["w_down"], *args,
                                          **opts)
    idx, w = moe.moe_route_sigmoid_grouped(wl["logits"], *args, **opts)
    d = moe.moe_dispatch(wl["x"], idx, wl["E"])
    y = moe.moe_experts_forward(d["xd"], d["offsets"], wl["w_gate"],
                                wl["w_up"], wl["w_down"])
    staged = moe.moe_combine(y, w, d["token_row"])
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), staged.view(torch.int16))


def test_full_size_sampled_tokens():
    """The grouped workload at full size (T=8192, H=7168, I=2048, E=64), in
    the launch configuration the benchmark times; sampled output tokens
    computed one by one by the oracle."""
    wl = workloads.make("grouped", device="cuda")
    T = wl["T"]
    print("case: grouped full size", flush=True)
    out = moe.moe_forward_sigmoid_grouped(
        wl["x"], wl["logits"], wl["w_gate"], wl["w_up"], wl["w_down"],
        wl["k"], wl["groups"], wl["selected_groups"], bias=wl["bias"],
        group_top_two=wl["group_top_two"], renormalize=wl["renorm"],
        scale=wl["scale"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    tokens = sorted({0, T - 1, *rng.choice(T, size=6, replace=False)})
    _, _, ref = forward_sigmoid_tokens(
        _np(wl, "x"), _np(wl, "logits"), wl["bias"].cpu().numpy(),
        _np(wl, "w_gate"), _np(wl, "w_up"), _np(wl, "w_down"), wl["k"],
        wl["groups"], wl["selected_groups"], wl["group_top_two"],
        wl["renorm"], wl["scale"], "bf16", tokens)
    got = values(out[torch.tensor(tokens, device="cuda")])
    assert_close(got, ref, "bf16", "grouped T=%d" % T)

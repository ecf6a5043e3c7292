"""GPU parity of moe_experts_forward_clipped (the clipped SwiGLU activation
of the MindSpeed-Ops page's clipped_swiglu in the gate+up epilogue) against
the oracle: every kernel path (prefill tiles, decode tiles, the FMA path)
with limits that clamp often, fed the oracle's dispatched rows."""

import numpy as np
import pytest
import torch

import mixture_experts_layer_28_amd as moe
from mixture_experts_layer_28_amd import workloads
from oracle.fp import round_to
from oracle.moe import dispatch, experts, route
from parity_util import assert_close, values

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tensor(vals, fmt):
    return torch.from_numpy(np.asarray(vals, dtype=np.float32)).to(TDT[fmt])


def _u32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(
        np.int32))


# (T, H, I, E, k, fmt): prefill tiles (N >= 96 E), decode tiles, fp32 and
# K % 8 != 0 on the FMA path
SHAPES = [(600, 256, 384, 4, 2, "bf16"), (300, 136, 200, 5, 2, "f16"),
          (20, 512, 384, 64, 8, "bf16"), (64, 128, 256, 8, 2, "f32"),
          (130, 100, 60, 6, 2, "bf16")]


@pytest.mark.parametrize("T,H,I,E,k,fmt", SHAPES)
@pytest.mark.parametrize("alpha,limit", [(1.702, 7.0), (1.702, 0.75),
                                         (0.5, 0.25), (1.702, 0.0)])
def test_clipped_experts(T, H, I, E, k, fmt, alpha, limit):
    rng = np.random.default_rng(T + E)
    # unit-scale gate and up values (as the other expert tests use), so a
    # limit of 0.75 clamps about a quarter of them and 0 all of them
    x = round_to(rng.standard_normal((T, H)), fmt)
    lg = round_to(rng.standard_normal((T, E)), fmt)
    wg = round_to(rng.standard_normal((E, I, H)) / np.sqrt(H), fmt)
    wu = round_to(rng.standard_normal((E, I, H)) / np.sqrt(H), fmt)
    wd = round_to(rng.standard_normal((E, H, I)) / np.sqrt(I), fmt)
    idx, _ = route(lg, k, True, fmt)
    d = dispatch(x, idx, E)
    print("case: clipped T=%d E=%d %s L=%g" % (T, E, fmt, limit), flush=True)
    y = moe.moe_experts_forward_clipped(
        _tensor(d["xd"], fmt).cuda(), _u32(d["offsets"]).cuda(),
        _tensor(wg, fmt).cuda(), _tensor(wu, fmt).cuda(),
        _tensor(wd, fmt).cuda(), alpha=alpha, limit=limit)
    torch.cuda.synchronize()
    want = experts(d["xd"], d["offsets"], wg, wu, wd, fmt,
                   clip=(alpha, limit))
    assert_close(values(y), want, fmt, "clipped %s L=%g" % (fmt, limit))


def test_full_size_sampled_rows():
    """The Mixtral-shaped layer's expert stage with the page's defaults
    (alpha 1.702, limit 7) in the benchmark's launch configuration, and a
    limit of 0.05 that clamps most values; sampled dispatched rows computed
    one by one by the oracle."""
    wl = workloads.make("mixtral", device="cuda")
    idx, _ = moe.moe_route(wl["logits"], wl["k"], True)
    d = moe.moe_dispatch(wl["x"], idx, wl["E"])
    off = d["offsets"].cpu().numpy().view(np.uint32).astype(np.int64)
    rng = np.random.default_rng(4)
    N = d["xd"].shape[0]
    rows = sorted({0, N - 1, *rng.choice(N, size=6, replace=False)})
    for alpha, limit in ((1.702, 7.0), (1.702, 0.05)):
        print("case: clipped mixtral L=%g" % limit, flush=True)
        y = moe.moe_experts_forward_clipped(d["xd"], d["offsets"],
                                            wl["w_gate"], wl["w_up"],
                                            wl["w_down"], alpha, limit)
        torch.cuda.synchronize()
        for r in rows:
            e = int(np.searchsorted(off, r, side="right") - 1)
            one = np.array([0, 1])
            tn = lambda t: workloads.to_numpy(t, "bf16")  # noqa: E731
            want = experts(tn(d["xd"][r:r + 1]), one,
                           tn(wl["w_gate"][e:e + 1]), tn(wl["w_up"][e:e + 1]),
                           tn(wl["w_down"][e:e + 1]), "bf16",
                           clip=(alpha, limit))
            assert_close(values(y[r:r + 1]), want, "bf16",
                         "row %d L=%g" % (r, limit))


def test_forward_clipped_one_call_equals_staged():
    """moe_forward_clipped is route -> dispatch -> clipped experts ->
    combine on one stream, bit for bit, and matches the oracle."""
    wl = workloads.make("edge", T=300, H=128, I=192, E=8, k=2)
    wl["logits"] = torch.nan_to_num(wl["logits"].float(), nan=0.0,
                                    posinf=4.0, neginf=-4.0)
    c = {key: wl[key].to(torch.bfloat16).cuda()
         for key in ("x", "logits", "w_gate", "w_up", "w_down")}
    one = moe.moe_forward_clipped(c["x"], c["logits"], c["w_gate"],
                                  c["w_up"], c["w_down"], 2, True, 1.702,
                                  0.5)
    idx, w = moe.moe_route(c["logits"], 2, True)
    d = moe.moe_dispatch(c["x"], idx, 8)
    y = moe.moe_experts_forward_clipped(d["xd"], d["offsets"], c["w_gate"],
                                        c["w_up"], c["w_down"], 1.702, 0.5)
    staged = moe.moe_combine(y, w, d["token_row"])
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), staged.view(torch.int16))
    tn = lambda t: workloads.to_numpy(t.cpu(), "bf16")  # noqa: E731
    idx_r, w_r = route(tn(c["logits"]), 2, True, "bf16")
    d_r = dispatch(tn(c["x"]), idx_r, 8)
    y_r = experts(d_r["xd"], d_r["offsets"], tn(c["w_gate"]), tn(c["w_up"]),
                  tn(c["w_down"]), "bf16", clip=(1.702, 0.5))
    from oracle.moe import combine
    out_r = combine(y_r, w_r, d_r["token_row"], "bf16")
    assert_close(values(one), out_r, "bf16", "forward clipped")

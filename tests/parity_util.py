"""Comparison rules for GPU-vs-oracle parity.

Tolerances (stated once, used by every parity test):
* indices, offsets, segment membership, row mappings: bit exact;
* fp32 values: max_i |a_i - b_i| / max(|b_i|, rms(b)) <= 1e-4 (the rms floor
  keeps outputs that cancel to near zero from dominating);
* fp16 / bf16 values: |a - b| <= 1e-2 + 2e-2 * |b| elementwise;
* NaN positions must agree exactly (NaN compares equal to NaN).
"""

import numpy as np
import torch

from oracle.fp import decode
from mixture_experts_layer_28_amd.workloads import to_numpy

FMT_OF = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def values(t):
    """A torch tensor -> float64 numpy values (exact), decoded by the
    oracle's own format decoder."""
    fmt = FMT_OF[t.dtype]
    return decode(to_numpy(t, fmt), fmt)


def u32(t):
    """An int32 index tensor -> numpy uint32 (same bits)."""
    return t.detach().cpu().numpy().view(np.uint32)


def assert_close(got, want, fmt, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), "%s: NaN positions differ (%d vs %d)" % (
        what, gn.sum(), wn.sum())
    ok = ~wn
    g, w = got[ok], want[ok]
    if g.size == 0:
        return
    inf = np.isinf(w) | np.isinf(g)
    assert np.array_equal(g[inf], w[inf]), "%s: infinities differ" % what
    g, w = g[~inf], w[~inf]
    if g.size == 0:
        return
    if fmt == "f32":
        rms = np.sqrt(np.mean(w * w))
        err = np.abs(g - w) / np.maximum(np.abs(w), max(rms, 1e-30))
        worst = float(err.max())
        assert worst <= 1e-4, "%s: fp32 rel err %.3g > 1e-4" % (what, worst)
    else:
        lim = 1e-2 + 2e-2 * np.abs(w)
        bad = np.abs(g - w) > lim
        assert not bad.any(), "%s: %d of %d beyond 1e-2 + 2e-2|b| (worst " \
            "excess %.3g)" % (what, bad.sum(), bad.size,
                              float((np.abs(g - w) - lim).max()))


def assert_dispatch_matches(gpu, ref, idx, E, x_bits=None):
    """gpu: dict of torch tensors from moe_dispatch; ref: oracle dispatch
    dict; idx: [T,k] uint32 routing table both were built from."""
    T, k = idx.shape
    N = T * k
    off = u32(gpu["offsets"]).astype(np.int64)
    np.testing.assert_array_equal(off, ref["offsets"])
    rex = u32(gpu["row_expert"])
    np.testing.assert_array_equal(rex, ref["row_expert"])
    rtok = u32(gpu["row_token"])
    trow = u32(gpu["token_row"]).reshape(T, k)
    # the stored mapping: a bijection onto [0, N) consistent with idx
    assert np.array_equal(np.sort(trow.ravel()), np.arange(N, dtype=np.uint32))
    np.testing.assert_array_equal(rex[trow.ravel()], idx.ravel())
    np.testing.assert_array_equal(
        rtok[trow.ravel()], np.repeat(np.arange(T, dtype=np.uint32), k))
    # per-expert token multisets (the contract), then the stable order this
    # library documents (equal to the oracle's (token, slot) order)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        np.testing.assert_array_equal(np.sort(rtok[lo:hi]),
                                      np.sort(ref["row_token"][lo:hi]))
    np.testing.assert_array_equal(rtok, ref["row_token"])
    np.testing.assert_array_equal(trow, ref["token_row"])
    if x_bits is not None:
        xd = gpu["xd"].detach().cpu()
        if xd.dtype == torch.float32:
            xd_bits = xd.numpy().view(np.uint32)
        else:
            xd_bits = xd.view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(xd_bits, x_bits[rtok])

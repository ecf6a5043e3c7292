"""Pins for the oracle's clipped SwiGLU activation (oracle.moe.clipped_silu_times
and the ``clip`` option of oracle.moe.experts).

Source: the MindSpeed-Ops page's ``clipped_swiglu`` parameter table
(swiglu_alpha default 1.702; swiglu_limit L >= 0 default 7; gate clamped
from above at L, up clamped to [-L, L]).  Pins:
* alpha = 1 with an infinite limit is the plain SwiGLU, and the clipped
  experts then equal the pinned plain experts bit for bit;
* torch in float64 (clamp, sigmoid) on random values around the limits;
* closed forms at the clamps: a gate at or above L acts as L, an up value
  beyond L acts as +-L; a zero gate gives zero;
* NaN propagates through the clamps.
"""

import math

import numpy as np
import torch

from oracle.fp import round_to
from oracle.moe import clipped_silu_times, experts, silu_times


def test_reduces_to_plain_swiglu():
    rng = np.random.default_rng(1)
    g = rng.standard_normal(1000) * 5
    u = rng.standard_normal(1000) * 5
    assert np.array_equal(clipped_silu_times(g, u, 1.0, np.inf),
                          silu_times(g, u))
    T, H, I, E = 30, 8, 12, 3
    xd = round_to(rng.standard_normal((T, H)), "bf16")
    off = np.array([0, 10, 10, 30])
    wg, wu, wd = (round_to(rng.standard_normal(s) * 0.5, "bf16")
                  for s in ((E, I, H), (E, I, H), (E, H, I)))
    assert np.array_equal(experts(xd, off, wg, wu, wd, "bf16",
                                  clip=(1.0, np.inf)),
                          experts(xd, off, wg, wu, wd, "bf16"))


def test_matches_torch():
    rng = np.random.default_rng(2)
    g = rng.standard_normal(5000) * 8
    u = rng.standard_normal(5000) * 8
    for alpha, limit in ((1.702, 7.0), (1.0, 0.5), (2.5, 0.0)):
        G, U = torch.tensor(g), torch.tensor(u)
        gc = torch.clamp(G, max=limit)
        uc = torch.clamp(U, min=-limit, max=limit)
        want = (gc * torch.sigmoid(alpha * gc) * uc).numpy()
        got = clipped_silu_times(g, u, alpha, limit)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-300)


def test_closed_forms_at_the_clamps():
    a, L = 1.702, 7.0
    s = 1.0 / (1.0 + math.exp(-a * L))
    got = clipped_silu_times(np.array([7.0, 9.0, 100.0, 0.0]),
                             np.array([1.0, 8.0, -50.0, 3.0]), a, L)
    assert got[0] == L * s * 1.0
    assert got[1] == L * s * L
    assert got[2] == L * s * -L
    assert got[3] == 0.0
    # below the limit the gate is untouched: swish with parameter alpha
    g = -3.0
    assert clipped_silu_times(np.array([g]), np.array([2.0]), a, L)[0] == \
        g * 2.0 / (1.0 + math.exp(-a * g))


def test_nan_propagates():
    got = clipped_silu_times(np.array([np.nan, 1.0]),
                             np.array([1.0, np.nan]), 1.702, 7.0)
    assert np.isnan(got).all()

"""Pins for the oracle's storage-format rounding (oracle.fp).

round_to is written from the IEEE 754 definition of roundTiesToEven for a
generic binary format.  It is pinned against library casts that implement
the same rule (numpy's float64->float16 and float64->float32 conversions,
torch's float32->bfloat16 conversion) and against boundary values worked out
by hand (ties, subnormals, overflow).
"""

import numpy as np
import pytest
import torch

from oracle.fp import decode, encode_bits, round_to


def _probe_values(n=200_000, seed=7):
    rng = np.random.default_rng(seed)
    parts = [
        rng.standard_normal(n),
        rng.standard_normal(n) * 1e4,
        rng.standard_normal(n) * 1e-6,
        np.ldexp(rng.uniform(0.5, 1.0, n), rng.integers(-160, 140, n)),
        -np.ldexp(rng.uniform(0.5, 1.0, n), rng.integers(-160, 140, n)),
    ]
    return np.concatenate(parts)


def test_f16_matches_numpy_cast():
    x = _probe_values()
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)
    got = round_to(x, "f16")
    np.testing.assert_array_equal(got, want)


def test_f32_matches_numpy_cast():
    x = _probe_values()
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).astype(np.float64)
    got = round_to(x, "f32")
    np.testing.assert_array_equal(got, want)


def test_bf16_matches_torch_cast_on_float32_inputs():
    # From binary32 inputs a single rounding is all that happens, so torch's
    # float32 -> bfloat16 cast (round to nearest even) is the reference.
    with np.errstate(over="ignore"):
        x = _probe_values().astype(np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_to(x.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("fmt,val,want", [
    # ties to even at 1.0: the quantum is 2**-7 (bf16), 2**-10 (f16)
    ("bf16", 1.0 + 2.0 ** -8, 1.0),
    ("bf16", 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),
    ("f16", 1.0 + 2.0 ** -11, 1.0),
    ("f16", 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),
    # largest finite values, and the halfway point above them overflows
    ("f16", 65504.0, 65504.0),
    ("f16", 65519.99, 65504.0),
    ("f16", 65520.0, np.inf),
    ("bf16", (2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),
    ("bf16", (2 - 2.0 ** -7 + 2.0 ** -9) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),
    ("bf16", (2 - 2.0 ** -8) * 2.0 ** 127, np.inf),
    # smallest subnormals and ties below them
    ("f16", 2.0 ** -24, 2.0 ** -24),
    ("f16", 2.0 ** -25, 0.0),
    ("f16", 3 * 2.0 ** -26, 2.0 ** -24),
    ("bf16", 2.0 ** -133, 2.0 ** -133),
    ("bf16", 2.0 ** -134, 0.0),
    ("bf16", 3 * 2.0 ** -135, 2.0 ** -133),
    ("f32", 2.0 ** -149, 2.0 ** -149),
    ("f32", 2.0 ** -150, 0.0),
])
def test_boundaries(fmt, val, want):
    assert round_to(np.array([val]), fmt)[0] == want
    assert round_to(np.array([-val]), fmt)[0] == -want


def test_specials_pass_through():
    x = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0])
    for fmt in ("f32", "f16", "bf16"):
        r = round_to(x, fmt)
        assert np.isnan(r[0]) and r[1] == np.inf and r[2] == -np.inf
        assert r[3] == 0.0 and not np.signbit(r[3]) and np.signbit(r[4])


def test_bf16_bits_round_trip():
    x = round_to(_probe_values(5000), "bf16")
    x = x[np.isfinite(x)]
    bits = encode_bits(x, "bf16")
    np.testing.assert_array_equal(decode(bits, "bf16"), x)
    t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    np.testing.assert_array_equal(
        t.view(torch.int16).numpy().view(np.uint16), bits)

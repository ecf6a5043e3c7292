"""Floating-point formats for the oracle (test infrastructure only).

The MoE contract in the ruDNN user guide (section 4, routing contract, and
section 5, expert weights and dispatch) admits F32, F16 and BF16 tensors.  The
oracle works on float64 numbers and needs two things from the formats:

* decoding stored values into float64 (always exact), and
* rounding a float64 result to the nearest value of a storage format with
  ties to even, which is the IEEE 754 default rounding attribute
  (roundTiesToEven), including subnormals and overflow to infinity.

``round_to`` is written from that definition for a generic binary format with
``p`` significand bits (implicit bit included), minimum normal exponent
``emin`` and maximum exponent ``emax``; it is pinned against numpy's float16
and float32 casts and against hand-picked boundary values.
"""

import numpy as np

# name -> (significand bits p incl. the implicit bit, emin, emax)
FORMATS = {
    "f32": (24, -126, 127),
    "f16": (11, -14, 15),
    "bf16": (8, -126, 127),
}

BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def round_to(x, fmt):
    """Round float64 ``x`` to the nearest ``fmt`` value, ties to even.

    Returns float64 holding exactly representable ``fmt`` values.  NaN stays
    NaN, infinities stay, and magnitudes that round past the largest finite
    value become infinities of the same sign.
    """
    p, emin, emax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x)
    xf = x[fin]
    # x = m * 2**q with 0.5 <= |m| < 1, so the leading bit has weight 2**(q-1).
    _, q = np.frexp(xf)
    # Below the normal range the quantum stops shrinking (gradual underflow).
    lead = np.maximum(q - 1, emin)
    shift = lead - (p - 1)                    # the quantum is 2**shift
    scaled = np.ldexp(xf, -shift)             # exact: a power-of-two scale
    r = np.ldexp(np.rint(scaled), shift)      # np.rint rounds ties to even
    over = np.abs(r) >= np.ldexp(1.0, emax + 1)
    r[over] = np.copysign(np.inf, xf[over])
    out[fin] = r
    return out


def decode(a, fmt):
    """Stored values -> float64 (exact).

    ``a`` may be a float64/float32/float16 array holding values of ``fmt``,
    or, for ``bf16``, a uint16 array of raw bit patterns (sign, 8 exponent
    bits, 7 fraction bits: the upper half of a binary32 word).
    """
    a = np.asarray(a)
    if fmt == "bf16" and a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if fmt == "f16" and a.dtype == np.uint16:
        return a.view(np.float16).astype(np.float64)
    if fmt == "f32" and a.dtype == np.uint32:
        return a.view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def encode_bits(x, fmt):
    """float64 values already representable in ``fmt`` -> raw bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    if fmt == "f32":
        return x.astype(np.float32).view(np.uint32)
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    # bf16: a representable value is a binary32 whose low 16 bits are zero.
    b = x.astype(np.float32).view(np.uint32)
    return (b >> 16).astype(np.uint16)

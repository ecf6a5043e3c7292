"""Seeded synthetic inputs shaped like the MoE workloads.

This module draws random numbers and nothing else: it holds none of the MoE
arithmetic.  Tests, the smoke check and the benchmark use it to build the
same inputs for the HIP library and for the CPU oracle.

Workloads (sizes: T tokens, H hidden, I intermediate, E experts, k top-k):

* ``tiny``   fp32, T=64,  H=128,  I=256,   E=8,   k=2, renormalised
* ``edge``   fp16, T=512, H=256,  I=512,   E=16,  k in {1,4,16}, both renorm
             settings; logits on a 0.5 grid (forces ties) with 25 rows
             holding a NaN, 25 holding a +inf and 25 that are all -inf
* ``mixtral`` bf16, T=4096, H=4096, I=14336, E=8,  k=2, renormalised
* ``fine``   bf16, T=8192, H=7168, I=2048,  E=64,  k=8, renormalised; a
             per-expert logit bias (std 2) skews the load so that some
             experts receive no token
* ``decode`` bf16, T=32 or 256, H=4096, I=1536, E=128, k=8, not renormalised
* ``grouped`` bf16, the ``fine`` layer shape (T=8192, H=7168, I=2048, E=64,
             k=8) under group-limited sigmoid routing: 8 groups of 8
             experts, 4 groups kept, group score = sum of the two largest,
             renormalised, scale 2.5, FP32 correction bias N(0, 0.25)

Distributions: "N(0, s)" means standard deviation s.  Inputs and logits are
N(0,1).  ``tiny`` and ``edge`` draw gate/up with std 1/sqrt(H) and down with
std 1/sqrt(I); the bf16 workloads use std 0.02 for every expert weight.

Random streams: workload number c (tiny=1 ... grouped=6) seeds
``numpy.random.SeedSequence(1000 + c)`` and spawns one child per tensor
(x, logits, gate, up, down, bias, edge rows).  x, logits, bias and the edge
rows come from numpy PCG64 in float32 and are rounded to the storage dtype
by torch (round to nearest even).  Expert weights of up to 2**24 elements come
from the same numpy streams; larger ones are drawn with torch's generator on
the target device (seeded from the tensor's child seed), one expert at a
time, because a CPU draw of billions of normals takes minutes.
"""

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16,
               "bf16": torch.bfloat16}

WORKLOADS = {
    "tiny": dict(num=1, fmt="f32", T=64, H=128, I=256, E=8, k=2, renorm=True,
                 w_std="fan_in"),
    "edge": dict(num=2, fmt="f16", T=512, H=256, I=512, E=16, k=4,
                 renorm=True, w_std="fan_in", ks=(1, 4, 16),
                 renorms=(True, False)),
    "mixtral": dict(num=3, fmt="bf16", T=4096, H=4096, I=14336, E=8, k=2,
                    renorm=True, w_std=0.02),
    "fine": dict(num=4, fmt="bf16", T=8192, H=7168, I=2048, E=64, k=8,
                 renorm=True, w_std=0.02, bias_std=2.0),
    "decode": dict(num=5, fmt="bf16", T=32, H=4096, I=1536, E=128, k=8,
                   renorm=False, w_std=0.02, Ts=(32, 256)),
    "grouped": dict(num=6, fmt="bf16", T=8192, H=7168, I=2048, E=64, k=8,
                    renorm=True, w_std=0.02, groups=8, selected_groups=4,
                    group_top_two=True, scale=2.5, corr_bias_std=0.25),
}

EDGE_ROWS = 25          # floor(0.05 * 512) rows of each poisoned kind
NUMPY_LIMIT = 1 << 24   # larger expert weights are drawn on the device


def _streams(num):
    kids = np.random.SeedSequence(1000 + num).spawn(7)
    names = ("x", "logits", "gate", "up", "down", "bias", "edge")
    return dict(zip(names, kids))


def _normal(seed_seq, shape):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    return rng.standard_normal(shape, dtype=np.float32)


def _weights(seed_seq, E, rows, cols, std, fmt, device):
    tdt = TORCH_DTYPE[fmt]
    if E * rows * cols <= NUMPY_LIMIT:
        w = _normal(seed_seq, (E, rows, cols)) * np.float32(std)
        return torch.from_numpy(w).to(tdt).to(device)
    out = torch.empty((E, rows, cols), dtype=tdt, device=device)
    seed = int(seed_seq.generate_state(1, dtype=np.uint64)[0] & ((1 << 62) - 1))
    gen = torch.Generator(device=device).manual_seed(seed)
    for e in range(E):
        chunk = torch.randn((rows, cols), generator=gen, device=device,
                            dtype=torch.float32)
        out[e].copy_((chunk * std).to(tdt))
    return out


def make(name, device="cpu", T=None, k=None, renorm=None, H=None, I=None,
         E=None):
    """Build one workload.  Keyword overrides shrink or vary it (tests use
    them for ragged and edge shapes); the default is the named workload.

    Returns a dict: x [T,H], logits [T,E], w_gate/w_up [E,I,H],
    w_down [E,H,I] (torch tensors on ``device``), bias (the float32
    correction bias [E] of group-limited routing, else None), plus k,
    renorm, fmt, the sizes and, for ``grouped``, the routing options.
    """
    cfg = dict(WORKLOADS[name])
    T = cfg["T"] if T is None else T
    H = cfg["H"] if H is None else H
    I = cfg["I"] if I is None else I
    E = cfg["E"] if E is None else E
    k = cfg["k"] if k is None else k
    renorm = cfg["renorm"] if renorm is None else renorm
    fmt = cfg["fmt"]
    tdt = TORCH_DTYPE[fmt]
    st = _streams(cfg["num"])

    x = torch.from_numpy(_normal(st["x"], (T, H))).to(tdt).to(device)

    z = _normal(st["logits"], (T, E))
    if name == "edge":
        z = (np.rint(np.float32(2.0) * z) / np.float32(2.0)).astype(np.float32)
        rng = np.random.Generator(np.random.PCG64(st["edge"]))
        n = min(EDGE_ROWS, T // 3)
        perm = rng.permutation(T)
        cols = rng.integers(0, E, size=2 * n)
        for i, t in enumerate(perm[:n]):
            z[t, cols[i]] = np.nan
        for i, t in enumerate(perm[n:2 * n]):
            z[t, cols[n + i]] = np.inf
        z[perm[2 * n:3 * n]] = -np.inf
    if "bias_std" in cfg:
        b = _normal(st["bias"], (E,)) * np.float32(cfg["bias_std"])
        z = (z + b[None, :]).astype(np.float32)
    logits = torch.from_numpy(z).to(tdt).to(device)
    corr_bias = None
    if "corr_bias_std" in cfg:
        corr_bias = torch.from_numpy(
            _normal(st["bias"], (E,)) * np.float32(cfg["corr_bias_std"])
        ).to(device)

    if cfg["w_std"] == "fan_in":
        sg, sd = 1.0 / np.sqrt(H), 1.0 / np.sqrt(I)
    else:
        sg = sd = cfg["w_std"]
    w_gate = _weights(st["gate"], E, I, H, sg, fmt, device)
    w_up = _weights(st["up"], E, I, H, sg, fmt, device)
    w_down = _weights(st["down"], E, H, I, sd, fmt, device)
    out = dict(x=x, logits=logits, w_gate=w_gate, w_up=w_up, w_down=w_down,
               k=k, renorm=renorm, fmt=fmt, T=T, H=H, I=I, E=E, name=name,
               bias=corr_bias)
    for key in ("groups", "selected_groups", "group_top_two", "scale"):
        if key in cfg:
            out[key] = cfg[key]
    return out


def to_numpy(t, fmt):
    """A torch tensor of ``fmt`` as a numpy array the oracle decodes:
    float32/float16 arrays, or raw uint16 bit patterns for bf16."""
    t = t.detach().cpu().contiguous()
    if fmt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()

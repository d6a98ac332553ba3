"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module holds no trellis arithmetic: it only draws random numbers.  Both sides of
every parity check receive the same host arrays produced here.

Workloads (all T = 256 weights per sequence, i.e. one 16x16 weight tile per sequence,
bitshift trellis L = 16, k = 2):
  * targets: i.i.d. N(0, 1) float32 -- the pages' own quality experiments quantise
    i.i.d. Gaussian 256-weight sequences, and a random Hadamard transform makes real
    weights approximately i.i.d. Gaussian, so synthetic N(0, 1) stands in for them;
  * curvature weights: log-normal(0, 1), w = float32(exp(z)) with z ~ N(0, 1) drawn in
    binary64.
Generator: numpy PCG64 with a fixed seed per workload.
"""
from __future__ import annotations

import numpy as np

T_DEFAULT = 256

# name -> (sequences, code, weighted, seed for targets, seed for weights)
WORKLOADS = {
    "enc16_1mad": dict(B=16, code="1mad", weighted=False, seed=1),
    "enc4096x4096_1mad": dict(B=65536, code="1mad", weighted=False, seed=2),
    "enc4096x14336_3inst": dict(B=229376, code="3inst", weighted=False, seed=3),
    "enc4096x4096_1mad_weighted": dict(B=65536, code="1mad", weighted=True, seed=4, wseed=40),
    "bcjr4096x4096_1mad": dict(B=65536, code="1mad", weighted=False, seed=5),
    "tb4096x4096_1mad": dict(B=65536, code="1mad", weighted=False, seed=6),
    "tb4096x14336_3inst": dict(B=229376, code="3inst", weighted=False, seed=7),
}


def targets(B: int, T: int = T_DEFAULT, seed: int = 0) -> np.ndarray:
    """[B][T] float32 i.i.d. N(0, 1)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal((B, T), dtype=np.float32)


def weights(B: int, T: int = T_DEFAULT, seed: int = 0) -> np.ndarray:
    """[B][T] float32 log-normal(0, 1) positive error weights."""
    g = np.random.Generator(np.random.PCG64(seed))
    z = g.standard_normal((B, T), dtype=np.float64)
    return np.exp(z).astype(np.float32)


def workload(name: str, B: int | None = None, T: int = T_DEFAULT):
    """(targets, weights or None, code) for a named workload; B overrides the size
    (the first B rows of the full workload's stream of rows)."""
    spec = WORKLOADS[name]
    nb = spec["B"] if B is None else B
    s = targets(nb, T, spec["seed"])
    w = weights(nb, T, spec["wseed"]) if spec["weighted"] else None
    return s, w, spec["code"]


# XOR-Trellis palette code (workload parameters, not method arithmetic): the page prints
# the palettes but not the four parity masks, so the workloads fix four 14-bit masks of
# 8 history bits each, linearly independent over GF(2) (every palette and shuffle bit
# depends on the history, and the four are jointly uniform over uniform histories).
# Narrower trellises keep the masks' low L - 2 bits.
XOR_MASKS = (0x2D35, 0x1ACB, 0x34AE, 0x0F53)
# targets for the XOR code are N(0, 1) times the RMS of the 16 printed palette values,
# sqrt(137 / 16), so that targets and code values have the same spread
XOR_TARGET_SCALE = 2.9261749


def xor_masks(L: int = 16) -> tuple:
    keep = (1 << (L - 2)) - 1
    return tuple(m & keep for m in XOR_MASKS)


def xor_targets(B: int, T: int = T_DEFAULT, seed: int = 0) -> np.ndarray:
    """[B][T] float32 N(0, 1) targets scaled to the XOR palettes' spread."""
    return (targets(B, T, seed) * np.float32(XOR_TARGET_SCALE)).astype(np.float32)

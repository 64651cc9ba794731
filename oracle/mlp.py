"""The gated-MLP join between the 7B / 65B-class MLP linears, in fp64.

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may import this.

The pages' workloads stop at the linears; the 7B MLP block and the 65B-class
stack chain gate and up into down the usual way for these model families:
H = silu(G) * U elementwise, silu(g) = g sigma(g), sigma(g) = 1 / (1 + e^-g).
Its backward, for the gradient dH arriving at H:

    dG = dH * U * silu'(g),  silu'(g) = sigma(g) (1 + g (1 - sigma(g)))
    dU = dH * silu(g)

(the derivative of g sigma(g) by the product rule, with
sigma' = sigma (1 - sigma)). Inputs are the exact fp64 values of the bf16
numbers the GPU read; the results are exact up to fp64 rounding.
"""

from __future__ import annotations

import numpy as np


def sigmoid(g) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    # e^-|g| never overflows; the two branches are the same function
    e = np.exp(-np.abs(g))
    return np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu_mul_fwd(G, U) -> np.ndarray:
    """H = silu(G) * U."""
    G, U = np.asarray(G, dtype=np.float64), np.asarray(U, dtype=np.float64)
    return G * sigmoid(G) * U


def silu_mul_bwd(G, U, dH):
    """(dG, dU) of H = silu(G) * U for the incoming dH."""
    G, U, dH = (np.asarray(t, dtype=np.float64) for t in (G, U, dH))
    sg = sigmoid(G)
    dG = dH * U * (sg * (1.0 + G * (1.0 - sg)))
    dU = dH * G * sg
    return dG, dU


def bf16_step(ref) -> np.ndarray:
    """One bf16 step (unit in the last place) at |ref|: 2^(e - 7) for
    2^e <= |ref| < 2^(e+1), and the smallest subnormal step 2^-133 below the
    normal range. A bf16 output rounded once from a value within a small
    fraction of a step of ref lies within one step of it."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    _, e = np.frexp(a)                     # a = m 2^e, 0.5 <= m < 1
    step = np.ldexp(np.ones_like(a), e - 8)
    return np.maximum(step, 2.0 ** -133)

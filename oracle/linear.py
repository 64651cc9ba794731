"""Frozen-base linear with a LoRA branch, forward and backward, in fp64.

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may import this.

Sources:
* "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev): the
  three-piece summary (the frozen 4-bit base is expanded to bf16 for the
  multiply; only the low-rank branch learns, the base gets no gradient) and
  the storage / compute / learning diagram (bf16 matmuls; gradients flow back
  into the adapter only).
* "What is QLoRA?" (qubittool.com), "Key Characteristics": gradients are
  propagated through the quantized weights; adapters are trained in full
  precision.
* "QLoRA Explained ..." (gamut.so), "Step 3: Configure and Apply LoRA
  Adapters" and "QLoRA Hyperparameter Quick Reference": rank r, alpha, no
  bias, LoRA dropout 0.05.

Notation: W' [N, K] is the dequantized bf16 weight (``oracle.nf4.dequant``),
X [M, K], A [r, K], B [N, r], dY [M, N]; s = alpha / r (reading: the usual
LoRA scale; the pages give r and alpha but no formula). Every operand is the
exact fp64 value of the bf16 (or fp32) number the GPU consumed, and each
product is one fp64 matrix multiply. The result is the exact real product up
to fp64 rounding; it is unique, unlike a GPU's fp32 accumulation order.
"""

from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def linear_fwd(X, Wd, A, B, s):
    """Y = X W'^T + s (X A^T) B^T and the saved T = X A^T.  Returns (Y, T)."""
    X, Wd, A, B = _f64(X), _f64(Wd), _f64(A), _f64(B)
    s = float(s)
    T = X @ A.T
    Y = X @ Wd.T + s * (T @ B.T)
    return Y, T


def linear_bwd(X, Wd, A, B, s, dY, T=None):
    """Gradients of <dY, Y> with W' frozen.

    U  = dY B
    dX = dY W' + s U A
    dA = s U^T X
    dB = s dY^T T,   T = X A^T (recomputed in fp64 unless given)
    There is no gradient for W'.  Returns (dX, dA, dB, U).
    """
    X, Wd, A, B, dY = _f64(X), _f64(Wd), _f64(A), _f64(B), _f64(dY)
    s = float(s)
    if T is None:
        T = X @ A.T
    T = _f64(T)
    U = dY @ B
    dX = dY @ Wd + s * (U @ A)
    dA = s * (U.T @ X)
    dB = s * (dY.T @ T)
    return dX, dA, dB, U


def adapter_grads(X, A, B, s, dY, T=None):
    """The adapter gradients of ``linear_bwd`` alone (no dX product):
    U = dY B, dA = s U^T X, dB = s dY^T T with T = X A^T.  Returns (dA, dB, U).
    Used where the full dX would be too large a product for the oracle and dX
    is checked on sampled rows instead."""
    X, A, B, dY = _f64(X), _f64(A), _f64(B), _f64(dY)
    s = float(s)
    if T is None:
        T = X @ A.T
    T = _f64(T)
    U = dY @ B
    dA = s * (U.T @ X)
    dB = s * (dY.T @ T)
    return dA, dB, U


def relerr(Z, Zref) -> float:
    """Relative Frobenius error ||Z - Zref||_F / ||Zref||_F, in fp64."""
    Z, Zref = _f64(Z), _f64(Zref)
    den = np.linalg.norm(Zref)
    num = np.linalg.norm(Z - Zref)
    return float(num / den) if den > 0 else float(num)


def bf16_floor(Zref) -> float:
    """relerr of Zref rounded once to bf16 (RNE): the least error a bf16 output
    can have. Reported beside every bf16 result."""
    z = np.asarray(Zref, dtype=np.float64)
    z32 = z.astype(np.float32)
    u = z32.view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    return relerr(r, z)


def fp16_floor(Zref) -> float:
    """relerr of Zref rounded once to fp16 (RNE, via ``oracle.nf4.fp16_round``):
    the least error an fp16 output can have."""
    from oracle.nf4 import fp16_round
    z = np.asarray(Zref, dtype=np.float64)
    return relerr(fp16_round(z.astype(np.float32)), z)


def linear_fwd_dropout(X, Wd, A, B, s, mask, keep_scale):
    """The forward with dropout on the adapter's input (reading: the usual
    inverted dropout of a LoRA branch; the pages give the rate, 0.05, not the
    formula). D = mask * keep_scale elementwise on X, mask in {0, 1} drawn by
    the caller, keep_scale = 1 / (1 - p):

        Y = X W'^T + s ((X . D) A^T) B^T

    The base sees the undropped X. Returns (Y, Td) with Td = (X . D) A^T."""
    X, Wd, A, B = _f64(X), _f64(Wd), _f64(A), _f64(B)
    D = _f64(mask) * float(keep_scale)
    s = float(s)
    Td = (X * D) @ A.T
    Y = X @ Wd.T + s * (Td @ B.T)
    return Y, Td


def linear_bwd_dropout(X, Wd, A, B, s, dY, mask, keep_scale):
    """Gradients of <dY, Y> for ``linear_fwd_dropout`` (W' frozen):

    U  = dY B
    dX = dY W' + s (U A) . D
    dA = s U^T (X . D)
    dB = s dY^T Td,   Td = (X . D) A^T
    Returns (dX, dA, dB, U)."""
    X, Wd, A, B, dY = _f64(X), _f64(Wd), _f64(A), _f64(B), _f64(dY)
    D = _f64(mask) * float(keep_scale)
    s = float(s)
    Xd = X * D
    U = dY @ B
    dX = dY @ Wd + s * ((U @ A) * D)
    dA = s * (U.T @ Xd)
    dB = s * (dY.T @ (Xd @ A.T))
    return dX, dA, dB, U


# --------------------------------------------------------------------------- element-wise error bounds
#
# What a bf16 (or fp16) output of an fp32-accumulated product of 16-bit
# operands may differ from the exact value, element by element. The products
# of two 16-bit numbers are exact in fp32; a sum of n of them, in any order
# and any grouping, carries at most gamma_n * sum |terms| of error with
# gamma_n = n u / (1 - n u), u = 2^-24 (the standard forward bound of
# floating-point summation; u is taken as 2^-23 below). The low-rank term enters as the hi/lo bf16 pair
# of s T (T itself an fp32 sum over the contraction): the pair misses s T by
# at most 2^-18 |s T| (hi is s T to half a bf16 step, 2^-9 relative; lo is the
# remainder to half a bf16 step of itself), and s T is one fp32 product.
# The output is the fp32 sum rounded once: at most half a step of the output
# type more, 2^-8 relative for bf16 (8 significant bits), 2^-11 for fp16
# (11 bits, plus 2^-25 absolute in its subnormal range). So, with S the sum
# of absolute terms,
#
#     |z - z_exact| <= E + u_out (|z_exact| + E) + a_out,
#     E = gamma_(n + slack) S + (2^-17 + 2^-23) |s| (|X| |A|^T) |B|^T.
#
# `slack` covers the few extra fp32 additions a kernel may make (split
# contraction partials added in order, the low-rank columns padded to 64).
# The bound is loose on purpose against the typical error but it holds
# element by element, so a single wrong output (a misplaced tile, a wrong
# code, a dropped low-rank term on a row) fails it where a global Frobenius
# norm would not notice.

# (2^-23, not 2^-24: also holds for an accumulator that truncates instead of
# rounding to nearest)
_U32 = 2.0 ** -23
_OUT = {"bf16": (2.0 ** -8, 0.0), "fp16": (2.0 ** -11, 2.0 ** -25)}


def _gamma(n: int) -> float:
    nu = n * _U32
    return nu / (1.0 - nu)


def _bound(Zref, S_main, S_lora, s, n, out, slack):
    u_out, a_out = _OUT[out]
    E = _gamma(n + slack) * (S_main + abs(s) * S_lora) + (2.0 ** -17 + 2.0 ** -23) * abs(s) * S_lora
    return E + u_out * (np.abs(_f64(Zref)) + E) + a_out


def fwd_error_bound(X, Wd, A, B, s, Yref, out: str = "bf16", mask=None, keep_scale: float = 1.0,
                    slack: int = 256):
    """Largest |Y - Yref| an fp32-accumulated forward may show, element by
    element ([M, N]); `mask` / `keep_scale` as in ``linear_fwd_dropout``."""
    aX, aW = np.abs(_f64(X)), np.abs(_f64(Wd))
    S_main = aX @ aW.T
    S_lora = 0.0
    if A is not None and np.size(A):
        aXl = aX if mask is None else aX * (_f64(mask) * abs(float(keep_scale)))
        S_lora = (aXl @ np.abs(_f64(A)).T) @ np.abs(_f64(B)).T
    return _bound(Yref, S_main, S_lora, float(s), aX.shape[1], out, slack)


def dx_error_bound(dY, Wd, A, B, s, dXref, out: str = "bf16", mask=None, keep_scale: float = 1.0,
                   slack: int = 256):
    """Largest |dX - dXref| an fp32-accumulated dX may show, element by
    element ([M, K]); with dropout the low-rank term is multiplied by
    mask * keep_scale elementwise, as in ``linear_bwd_dropout``."""
    adY, aW = np.abs(_f64(dY)), np.abs(_f64(Wd))
    S_main = adY @ aW
    S_lora = 0.0
    if A is not None and np.size(A):
        S_lora = (adY @ np.abs(_f64(B))) @ np.abs(_f64(A))
        if mask is not None:
            S_lora = S_lora * (_f64(mask) * abs(float(keep_scale)))
    return _bound(dXref, S_main, S_lora, float(s), adY.shape[1], out, slack)


def outside_bound(Z, Zref, bound) -> int:
    """How many elements of Z lie outside Zref +- bound (NaN counts)."""
    d = np.abs(_f64(Z) - _f64(Zref))
    return int(np.count_nonzero(~(d <= bound)))

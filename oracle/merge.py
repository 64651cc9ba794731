"""Adapter merge and unmerge for deployment, exact in fp64 with one final
rounding.

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may import this.

Sources (cited by page title and section):
* "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev), the two
  prices, price 2 (deployment friction): the adapter cannot be folded into
  the 4-bit base itself (no 4-bit level lies between the allowed ones), so
  it is merged onto a dequantized bf16 copy; then fine-tune, merge,
  quantize again, serve.
* "QLoRA vs LoRA: How Quantized Low-Rank Adaptation Reduces Memory for LLM
  Fine-Tuning" (instagit.com), question on converting back to full precision
  after training: merge the low-rank weights with the base and dequantize to
  a higher precision (fp16 or fp32).
* "QLoRA Explained ..." (gamut.so), "Step 5: Save and Merge Adapters".

What is computed (readings of the pages):
* merged[i, c] = round(W'[i, c] + s * sum_j B[i, j] A[j, c]) with W' the
  dequantized base (``oracle.nf4.dequant``) and s = alpha / r, the LoRA
  scale of the forward pass, so that X merged^T reproduces the trained
  layer's output up to the weights' rounding;
* the exact value is rounded once, to nearest-even, to the output type
  (bf16, or fp32 for the "higher precision" copy);
* unmerge removes the delta again from a bf16 merged weight:
  round_bf16(merged - s B A). It returns W' only where that rounding lands
  back on it (in general it does not: the merged copy was rounded).
"""

from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even), returned as fp64; finite
    normal-range input. A bf16 number has 8 significant bits, so with
    x = m 2^e (0.5 <= |m| < 1) the result is round(256 m) 2^(e-8)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0), e - 8)


def bf16_value_bits(v) -> np.ndarray:
    """Bit patterns of fp64 values that are bf16 numbers (exact)."""
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def delta(A, B, s) -> np.ndarray:
    """s * B A, [N, K], fp64 (each product of two bf16 numbers is exact)."""
    return float(s) * (np.asarray(B, dtype=np.float64) @ np.asarray(A, dtype=np.float64))


def merge_exact(Wd, A, B, s) -> np.ndarray:
    """W' + s B A before the final rounding."""
    return np.asarray(Wd, dtype=np.float64) + delta(A, B, s)


def adapter_merge(Wd, A, B, s, out: str = "bf16") -> np.ndarray:
    """Merged weight as fp64 values of the output type ('bf16' or 'fp32')."""
    z = merge_exact(Wd, A, B, s)
    if out == "bf16":
        return round_bf16(z)
    if out == "fp32":
        return z.astype(np.float32).astype(np.float64)
    raise ValueError(out)


def adapter_unmerge(Wm, A, B, s) -> np.ndarray:
    """round_bf16(merged - s B A) as fp64 values."""
    return round_bf16(np.asarray(Wm, dtype=np.float64) - delta(A, B, s))

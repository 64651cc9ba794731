"""AdamW step on the adapter (the "paged" 32-bit optimizer), in fp64.

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may import this.

Sources (cited by page title and section):
* "QLoRA Explained ..." (gamut.so), "Paged Optimizers": optimizer states
  (momentum, variance) move between GPU and CPU memory when memory spikes;
  "Step 4: Train with SFTTrainer" and "QLoRA Hyperparameter Quick Reference":
  the 32-bit paged AdamW optimizer, learning rate 2e-4, cosine schedule with
  warmup, gradient accumulation.
* "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev), paged
  optimizers: AdamW states in pinned CPU RAM; piece 3: only the adapter learns.

The pages name the optimizer but give no update formula. Reading: AdamW
with decoupled weight decay and bias correction, states m, v
in fp32 ("32-bit"), step t >= 1:
    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    theta <- theta - lr * ( (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps) + wd * theta )
with the old theta in the decay term. The learning rate of a step (the
schedule) is an input.
"""

from __future__ import annotations

import numpy as np


def adamw_step(theta, g, m, v, t: int, lr: float, b1: float = 0.9, b2: float = 0.999, eps: float = 1e-8,
               wd: float = 0.0):
    """One step, all fp64. Returns (theta, m, v)."""
    theta, g, m, v = (np.asarray(a, dtype=np.float64) for a in (theta, g, m, v))
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    mhat = m / (1.0 - b1 ** t)
    vhat = v / (1.0 - b2 ** t)
    theta = theta - lr * (mhat / (np.sqrt(vhat) + eps) + wd * theta)
    return theta, m, v


def cosine_lr(step: int, total: int, warmup: int, peak: float, floor: float = 0.0) -> float:
    """Cosine schedule with linear warmup: peak * step / warmup for step <= warmup,
    then floor + (peak - floor) (1 + cos(pi p)) / 2 with p the fraction of the
    remaining steps done."""
    if step <= warmup:
        return peak * step / max(warmup, 1)
    p = (step - warmup) / max(total - warmup, 1)
    return floor + (peak - floor) * 0.5 * (1.0 + np.cos(np.pi * min(p, 1.0)))

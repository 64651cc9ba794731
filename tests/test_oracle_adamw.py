"""Pins for the oracle's AdamW step (no GPU).

Pages: the 32-bit paged AdamW optimizer over the adapter only ("QLoRA
Explained ...", "Paged Optimizers", "Step 4", the quick reference; "QLoRA:
Quantized Low-Rank Adaptation", paged optimizers and piece 3).

Pinned against torch.optim.AdamW run in fp64 on the CPU (the library routine
for this update), a hand-worked first step, and the schedule's end points.
"""

import math

import numpy as np
import torch

from oracle import adamw


def test_matches_torch_adamw_in_fp64_over_several_steps():
    g = np.random.default_rng(2)
    n = 257
    theta0 = g.standard_normal(n) * 0.05
    grads = [g.standard_normal(n) * 10.0 ** g.uniform(-6, -1) for _ in range(6)]
    for wd in (0.0, 0.01):
        for lr in (2e-4, 1e-3):
            p = torch.nn.Parameter(torch.tensor(theta0, dtype=torch.float64))
            opt = torch.optim.AdamW([p], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd)
            th, m, v = theta0.copy(), np.zeros(n), np.zeros(n)
            for t, gr in enumerate(grads, start=1):
                p.grad = torch.tensor(gr, dtype=torch.float64)
                opt.step()
                th, m, v = adamw.adamw_step(th, gr, m, v, t, lr, wd=wd)
                st = opt.state[p]
                # torch forms m by linear interpolation: equal up to fp64 rounding
                assert np.allclose(th, p.detach().numpy(), rtol=1e-13, atol=1e-17)
                assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-18)
                assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-24)


def test_hand_worked_first_step():
    # t = 1: the bias-corrected moments are g and g^2, so the step is
    # lr * g / (|g| + eps) plus the decay lr * wd * theta
    th, m, v = adamw.adamw_step([1.0, -2.0], [0.5, -0.25], [0.0, 0.0], [0.0, 0.0], 1, 0.1, wd=0.5, eps=0.0)
    assert np.allclose(m, [0.05, -0.025], rtol=1e-15)
    assert np.allclose(v, [0.00025, 0.0000625], rtol=1e-14)
    assert np.allclose(th, [1.0 - 0.1 * (1.0 + 0.5), -2.0 - 0.1 * (-1.0 - 1.0)], rtol=1e-14)


def test_cosine_schedule_end_points():
    assert adamw.cosine_lr(0, 100, 10, 2e-4) == 0.0
    assert math.isclose(adamw.cosine_lr(5, 100, 10, 2e-4), 1e-4)
    assert math.isclose(adamw.cosine_lr(10, 100, 10, 2e-4), 2e-4)
    assert math.isclose(adamw.cosine_lr(55, 100, 10, 2e-4), 1e-4)
    assert abs(adamw.cosine_lr(100, 100, 10, 2e-4)) < 1e-20

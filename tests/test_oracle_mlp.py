"""Pins of ``oracle.mlp`` (the gated-MLP join silu(G) * U) against facts that
do not come from it: torch's fp64 autograd of its own silu, closed forms at
special points, a central finite difference, and the bf16 step it uses."""

import math

import numpy as np
import torch

from oracle import mlp


def test_matches_torch_autograd_in_fp64():
    rng = np.random.default_rng(3)
    g = rng.normal(0.0, 3.0, 5000)
    u = rng.normal(0.0, 1.0, 5000)
    dh = rng.normal(0.0, 1.0, 5000)
    tg = torch.tensor(g, requires_grad=True)
    tu = torch.tensor(u, requires_grad=True)
    h = torch.nn.functional.silu(tg) * tu
    h.backward(torch.tensor(dh))
    assert np.allclose(mlp.silu_mul_fwd(g, u), h.detach().numpy(), rtol=1e-14, atol=1e-300)
    dg, du = mlp.silu_mul_bwd(g, u, dh)
    assert np.allclose(dg, tg.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert np.allclose(du, tu.grad.numpy(), rtol=1e-14, atol=1e-300)


def test_closed_forms():
    # silu(0) = 0, silu'(0) = 1/2, sigma(0) = 1/2, sigma(-g) = 1 - sigma(g)
    assert mlp.silu_mul_fwd(0.0, 3.0) == 0.0
    dg, du = mlp.silu_mul_bwd(0.0, 1.0, 1.0)
    assert dg == 0.5 and du == 0.0
    g = np.linspace(-30, 30, 601)
    assert np.allclose(mlp.sigmoid(-g), 1.0 - mlp.sigmoid(g), rtol=0, atol=4e-16)  # 1 - x cancels
    # far right silu(g) -> g, far left silu(g) -> g e^g (no overflow at -745)
    assert mlp.silu_mul_fwd(40.0, 1.0) == 40.0
    assert math.isclose(float(mlp.silu_mul_fwd(-40.0, 1.0)), -40.0 * math.exp(-40.0), rel_tol=1e-12)
    assert np.isfinite(mlp.silu_mul_fwd(-745.0, 1.0))
    # silu'(g) = sigma(g) (1 + g (1 - sigma(g))) at g = 1 by hand
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    assert math.isclose(float(mlp.silu_mul_bwd(1.0, 1.0, 1.0)[0]), s1 * (1.0 + (1.0 - s1)), rel_tol=1e-15)


def test_derivative_against_central_difference():
    g = np.linspace(-8, 8, 161)
    h = 1e-6
    fd = (mlp.silu_mul_fwd(g + h, 1.0) - mlp.silu_mul_fwd(g - h, 1.0)) / (2 * h)
    dg, _ = mlp.silu_mul_bwd(g, np.ones_like(g), np.ones_like(g))
    assert np.allclose(dg, fd, rtol=0, atol=1e-8)


def test_bf16_step_is_one_unit_in_the_last_place():
    # bf16 has 8 significant bits: the step at [1, 2) is 2^-7, at [0.5, 1) 2^-8
    assert mlp.bf16_step(1.0) == 2.0 ** -7
    assert mlp.bf16_step(1.99) == 2.0 ** -7
    assert mlp.bf16_step(0.75) == 2.0 ** -8
    assert mlp.bf16_step(-3.0) == 2.0 ** -6
    # torch's own bf16 neighbours are one step apart
    for v in (1.0, 3.5, 1e-3, 7e5, 0.3):
        t = torch.tensor([v], dtype=torch.bfloat16)
        nxt = (t.view(torch.int16) + 1).view(torch.bfloat16).double().item()
        assert math.isclose(nxt - t.double().item(), float(mlp.bf16_step(t.double().item())), rel_tol=0)

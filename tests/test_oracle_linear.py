"""Pins for the oracle's forward and backward (no GPU).

Pages: the 4-bit base is expanded to bf16 and multiplied; a low-rank branch
is added; gradients flow through the quantized weights into the adapter only
("QLoRA: Quantized Low-Rank Adaptation", three-piece summary and the storage /
compute / learning diagram; "What is QLoRA?", "Key Characteristics").
"""

import numpy as np
import torch

from oracle import linear, nf4


def _case(m=24, n=40, k=128, r=6, seed=0):
    g = np.random.default_rng(seed)
    X = g.standard_normal((m, k))
    Wd = g.standard_normal((n, k)) * 0.02
    A = g.uniform(-1, 1, (r, k)) / np.sqrt(k)
    B = g.standard_normal((n, r)) * 0.01
    dY = g.standard_normal((m, n))
    return X, Wd, A, B, dY


def test_forward_and_backward_match_fp64_autograd():
    X, Wd, A, B, dY = _case()
    s = 2.5
    Y, T = linear.linear_fwd(X, Wd, A, B, s)
    dX, dA, dB, U = linear.linear_bwd(X, Wd, A, B, s, dY)
    tX = torch.tensor(X, requires_grad=True)
    tA = torch.tensor(A, requires_grad=True)
    tB = torch.tensor(B, requires_grad=True)
    tW = torch.tensor(Wd, requires_grad=True)
    tY = torch.nn.functional.linear(tX, tW) + s * torch.nn.functional.linear(
        torch.nn.functional.linear(tX, tA), tB)
    tY.backward(torch.tensor(dY))
    assert np.allclose(Y, tY.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(T, X @ A.T)
    # the base is frozen: the oracle returns no weight gradient at all
    assert len(linear.linear_bwd(X, Wd, A, B, s, dY)) == 4


def test_bilinear_directional_derivatives_are_exact():
    """L = <dY, Y> is linear in each of X, A, B separately, so a finite step
    equals eps * <grad, E> up to fp64 rounding, with no truncation term."""
    X, Wd, A, B, dY = _case(seed=1)
    s = 0.25
    g = np.random.default_rng(11)

    def L(X_, A_, B_):
        return float(np.sum(dY * linear.linear_fwd(X_, Wd, A_, B_, s)[0]))

    dX, dA, dB, _ = linear.linear_bwd(X, Wd, A, B, s, dY)
    base = L(X, A, B)
    for grad, which in ((dX, 0), (dA, 1), (dB, 2)):
        E = g.standard_normal(grad.shape)
        eps = 1e-3
        args = [X, A, B]
        args[which] = args[which] + eps * E
        lhs = L(*args) - base
        rhs = eps * float(np.sum(grad * E))
        assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(rhs))


def test_special_cases():
    g = np.random.default_rng(12)
    k, n, r = 64, 48, 4
    Wd = g.standard_normal((n, k)) * 0.02
    A = g.uniform(-1, 1, (r, k)) / 8
    B = g.standard_normal((n, r)) * 0.01
    s = 2.0
    # X = I: Y lists the effective weight, W'^T + s A^T B^T
    Y, _ = linear.linear_fwd(np.eye(k), Wd, A, B, s)
    assert np.allclose(Y, Wd.T + s * A.T @ B.T, rtol=0, atol=1e-15)
    # B = 0: the branch vanishes exactly and so does dA
    X = g.standard_normal((8, k))
    dY = g.standard_normal((8, n))
    Y0, _ = linear.linear_fwd(X, Wd, A, np.zeros_like(B), s)
    assert np.array_equal(Y0, X @ Wd.T)
    _, dA0, _, _ = linear.linear_bwd(X, Wd, A, np.zeros_like(B), s, dY)
    assert np.all(dA0 == 0)
    # dY = I: dX lists the effective weight, W' + s B A
    dXI, _, _, _ = linear.linear_bwd(np.zeros((n, k)), Wd, A, B, s, np.eye(n))
    assert np.allclose(dXI, Wd + s * B @ A, rtol=0, atol=1e-15)
    # r = 0: plain linear
    Yr, Tr = linear.linear_fwd(X, Wd, np.zeros((0, k)), np.zeros((n, 0)), s)
    assert np.array_equal(Yr, X @ Wd.T) and Tr.shape == (8, 0)


def test_relerr_and_bf16_floor():
    g = np.random.default_rng(13)
    Z = g.standard_normal((256, 256))
    assert linear.relerr(Z, Z) == 0.0
    fl = linear.bf16_floor(Z)
    # one RNE rounding to 8 significant bits: relative rms error ~ 2^-9 / sqrt(3) .. 2^-8
    assert 1e-3 < fl < 2e-3
    Zb = nf4.bf16_bits_to_f32(nf4.bf16_bits(Z.astype(np.float32)))
    assert abs(linear.relerr(Zb, Z) - fl) < 1e-6


def test_end_to_end_small_layer_tolerance_is_feasible():
    """The 2e-3 bar is above the floor of one bf16 rounding of Y, i.e. a GPU
    that accumulates in fp32 and rounds once can meet it."""
    g = np.random.default_rng(14)
    W = (g.standard_normal((96, 256)) * 0.02).astype(np.float32)
    q = nf4.NF4Weight(W)
    X = nf4.bf16_bits_to_f32(nf4.bf16_bits(g.standard_normal((32, 256)).astype(np.float32)))
    A = nf4.bf16_bits_to_f32(nf4.bf16_bits((g.uniform(-1, 1, (8, 256)) / 16).astype(np.float32)))
    B = nf4.bf16_bits_to_f32(nf4.bf16_bits((g.standard_normal((96, 8)) * 0.01).astype(np.float32)))
    Y, _ = linear.linear_fwd(X, q.dequant(), A, B, 2.0)
    assert linear.bf16_floor(Y) < 2e-3


def test_adapter_grads_equal_the_full_backward():
    rng = np.random.default_rng(21)
    M, N, K, r, s = 37, 29, 64, 5, 0.75
    X, Wd = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    A, B, dY = rng.standard_normal((r, K)), rng.standard_normal((N, r)), rng.standard_normal((M, N))
    _, dA, dB, U = linear.linear_bwd(X, Wd, A, B, s, dY)
    dA2, dB2, U2 = linear.adapter_grads(X, A, B, s, dY)
    assert np.array_equal(dA, dA2) and np.array_equal(dB, dB2) and np.array_equal(U, U2)

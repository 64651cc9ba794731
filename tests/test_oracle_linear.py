"""Pins for the oracle's forward and backward (no GPU).

Pages: the 4-bit base is expanded to bf16 and multiplied; a low-rank branch
is added; gradients flow through the quantized weights into the adapter only
("QLoRA: Quantized Low-Rank Adaptation", three-piece summary and the storage /
compute / learning diagram; "What is QLoRA?", "Key Characteristics").
"""

import numpy as np
import pytest
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


# --------------------------------------------------------------------------- element-wise error bounds

def _bf16(x):
    """torch's fp32 -> bf16 conversion (RNE), back as fp64 (a library routine,
    not the oracle's)."""
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _fp32_sum_in_order(terms, order):
    """Sequential fp32 sum of terms[..., j] over j in the given order."""
    acc = np.zeros(terms.shape[:-1], dtype=np.float32)
    for j in order:
        acc = (acc + terms[..., j].astype(np.float32)).astype(np.float32)
    return acc


def _bf16_inputs(m, n, k, r, seed, b_sigma=0.3):
    rng = np.random.default_rng(seed)
    X = _bf16(rng.normal(0, 1, (m, k)))
    W = _bf16(rng.normal(0, 0.02, (n, k)))
    A = _bf16(rng.uniform(-1, 1, (r, k)) / np.sqrt(k))
    B = _bf16(rng.normal(0, b_sigma, (n, r)))
    dY = _bf16(rng.normal(0, 1, (m, n)))
    return X, W, A, B, dY


def _gpu_like_forward(X, W, A, B, s, order):
    """A forward computed the way a GPU kernel may: bf16 products summed in
    fp32 in the given order over [X | hi | lo] . [W | B | B], where hi / lo
    are torch's bf16 of s T and of the remainder, T an fp32 sum; one bf16
    rounding at the end."""
    T = _fp32_sum_in_order(X[:, None, :] * A[None, :, :], range(X.shape[1]))
    sT = (np.float32(s) * T).astype(np.float32)
    hi = _bf16(sT)
    lo = _bf16(sT.astype(np.float64) - hi)
    P = np.concatenate([X, hi, lo], axis=1)
    Q = np.concatenate([W, B, B], axis=1)
    terms = P[:, None, :] * Q[None, :, :]
    perm = [j for j in order] + list(range(X.shape[1], P.shape[1]))
    return _bf16(_fp32_sum_in_order(terms, perm))


@pytest.mark.parametrize("order", ["forward", "reverse", "largest_first"])
def test_bound_holds_for_fp32_accumulation_in_any_order(order):
    """Y and dX computed with fp32 sums in three orders (the largest-magnitude
    terms first is the order that loses most) and the low-rank term entering
    as a bf16 hi/lo pair all lie inside the bound, element by element."""
    m, n, k, r, s = 6, 10, 768, 8, 2.0
    X, W, A, B, dY = _bf16_inputs(m, n, k, r, 11)
    Yr, _ = linear.linear_fwd(X, W, A, B, s)

    def order_of(P, Q):
        kk = P.shape[1]
        if order == "forward":
            return list(range(kk))
        if order == "reverse":
            return list(range(kk))[::-1]
        return list(np.argsort(-np.abs(P).sum(0) * np.abs(Q).sum(0)))

    Y = _gpu_like_forward(X, W, A, B, s, order_of(X, W))
    bnd = linear.fwd_error_bound(X, W, A, B, s, Yr)
    assert linear.outside_bound(Y, Yr, bnd) == 0
    # dX is the same shape of computation with dY, W^T, B^T, A^T
    dXr, _, _, _ = linear.linear_bwd(X, W, A, B, s, dY)
    Wt = W.T.copy()
    dX = _gpu_like_forward(dY, Wt, B.T.copy(), A.T.copy(), s, order_of(dY, Wt))
    assert linear.outside_bound(dX, dXr, linear.dx_error_bound(dY, W, A, B, s, dXr)) == 0
    # the plain rounding of the exact value also lies inside
    assert linear.outside_bound(_bf16(Yr), Yr, bnd) == 0


def test_bound_is_a_few_bf16_steps_for_short_contractions():
    """With a short contraction the bound is dominated by the output's own
    rounding: never more than 1.5 bf16 steps (3 x 2^-8 |Y|) plus a small
    absolute part."""
    X, W, A, B, _ = _bf16_inputs(8, 16, 64, 4, 12)
    Yr, _ = linear.linear_fwd(X, W, A, B, 1.0)
    bnd = linear.fwd_error_bound(X, W, A, B, 1.0, Yr, slack=0)
    S = np.abs(X) @ np.abs(W).T + (np.abs(X) @ np.abs(A).T) @ np.abs(B).T
    assert np.all(bnd <= 2.0 ** -8 * np.abs(Yr) * 1.0001 + 1e-4 * S)


def test_bound_catches_a_dropped_low_rank_term_and_a_wrong_code():
    m, n, k, r, s = 8, 12, 128, 8, 2.0
    X, W, A, B, dY = _bf16_inputs(m, n, k, r, 13)
    Yr, _ = linear.linear_fwd(X, W, A, B, s)
    bnd = linear.fwd_error_bound(X, W, A, B, s, Yr)
    # the forward without its low-rank term
    base = _bf16(X @ W.T)
    assert linear.outside_bound(base, Yr, bnd) > m * n // 2
    # with the workloads' small B: one weight of row 3 moved by a quarter of
    # the row's largest weight (an outer NF4 level step): column 3 of Y leaves
    # the bound where |x| is not small, the other columns stay inside
    X, W, A, B, dY = _bf16_inputs(m, n, k, r, 13, b_sigma=0.01)
    Yr, _ = linear.linear_fwd(X, W, A, B, s)
    bnd = linear.fwd_error_bound(X, W, A, B, s, Yr)
    W2 = W.copy()
    W2[3, 5] += 0.25 * np.abs(W[3]).max()
    Y2 = _bf16(linear.linear_fwd(X, W2, A, B, s)[0])
    outside = np.abs(Y2 - Yr) > bnd
    assert outside[:, 3].sum() >= m // 2 and outside[:, [0, 1, 2, 4]].sum() == 0
    # dX without the low-rank term
    dXr, _, _, _ = linear.linear_bwd(X, W, A, B, s, dY)
    assert linear.outside_bound(_bf16(dY @ W), dXr, linear.dx_error_bound(dY, W, A, B, s, dXr)) > m * k // 2


def test_bound_with_dropout_covers_the_masked_branch():
    m, n, k, r, s, kappa = 6, 10, 256, 8, 2.0, 1.0 / 0.95
    X, W, A, B, dY = _bf16_inputs(m, n, k, r, 14)
    mask = (np.random.default_rng(1).random((m, k)) >= 0.05).astype(np.uint8)
    Yr, _ = linear.linear_fwd_dropout(X, W, A, B, s, mask, kappa)
    Y = _gpu_like_forward(X, W, A, B, s * kappa, range(k))  # the branch without its mask
    bnd = linear.fwd_error_bound(X, W, A, B, s, Yr, mask=mask, keep_scale=kappa)
    assert linear.outside_bound(_bf16(Yr), Yr, bnd) == 0
    assert linear.outside_bound(Y, Yr, bnd) > 0
    dXr, _, _, _ = linear.linear_bwd_dropout(X, W, A, B, s, dY, mask, kappa)
    dbnd = linear.dx_error_bound(dY, W, A, B, s, dXr, mask=mask, keep_scale=kappa)
    assert linear.outside_bound(_bf16(dXr), dXr, dbnd) == 0
    # dropping the mask from the branch of dX is caught
    dXn, _, _, _ = linear.linear_bwd(X, W, A, B, s * kappa, dY)
    assert linear.outside_bound(_bf16(dXn), dXr, dbnd) > 0

"""Pins for the oracle's NF4 codebook (no GPU).

What the pages fix: 16 levels, quantiles of a normal distribution, largest
magnitude 1 ("QLoRA: Quantized Low-Rank Adaptation", three-piece summary and
"NF4: a 4-bit format matched to weight statistics"; "QLoRA Explained ...",
"4-Bit NormalFloat (NF4) Quantization"). The exact zero comes from the
reading recorded in the oracle header (R1). NF4 must beat an evenly spaced
4-bit grid on bell-curve data ("NF4: a 4-bit format ...", last paragraph).
"""

import math

import numpy as np

from oracle import nf4


def _phi_inv_bisect(p: float) -> float:
    """An independent inverse normal CDF: bisection on 1/2 erfc(-x/sqrt 2)."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_sixteen_levels_sorted_with_exact_endpoints_and_zero():
    L = nf4.nf4_levels()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L.astype(np.float64)) > 0)
    assert L[0] == np.float32(-1.0) and L[15] == np.float32(1.0)
    assert L[7] == np.float32(0.0) and not np.signbit(L[7])
    # 7 negative, 8 positive: the larger half is positive (reading R1)
    assert (L < 0).sum() == 7 and (L > 0).sum() == 8


def test_levels_match_independent_inverse_cdf():
    """Rebuild the table with bisection on erfc (shares nothing with the
    stdlib inverse CDF the oracle uses) and demand the same fp32 bits."""
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    top = _phi_inv_bisect(delta)
    pos = [_phi_inv_bisect(0.5 + j / 8 * (delta - 0.5)) / top for j in range(1, 9)]
    neg = [-_phi_inv_bisect(0.5 + j / 7 * (delta - 0.5)) / top for j in range(1, 8)]
    ref = np.array(sorted(neg + [0.0] + pos)).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), nf4.nf4_levels().view(np.uint32))


def test_levels_are_far_from_fp32_rounding_boundaries():
    """Each fp64 level sits well inside its fp32 rounding interval, so any
    inverse CDF with relative error < 1e-9 rounds to the same table."""
    L64 = np.array(nf4.nf4_levels_fp64())
    L32 = L64.astype(np.float32)
    for v64, v32 in zip(L64, L32):
        if v64 == 0.0 or abs(v64) == 1.0:
            continue
        ulp = float(np.spacing(np.float32(abs(v32))))
        dist_to_edge = ulp / 2 - abs(v64 - float(v32))
        assert dist_to_edge / ulp > 0.02
        assert abs(v64) * 1e-9 < dist_to_edge


def test_levels_are_normal_quantiles_up_to_one_scale():
    """Positive levels times Phi^-1(delta) are the normal quantiles of evenly
    spaced probabilities: check Phi(level * top) against those probabilities
    with the erfc-based CDF, not the inverse the oracle used."""
    L = np.array(nf4.nf4_levels_fp64())
    delta = nf4.nf4_delta()
    top = _phi_inv_bisect(delta)
    cdf = [0.5 * math.erfc(-v * top / math.sqrt(2.0)) for v in L]
    pos = cdf[8:]
    neg = cdf[:7]
    for j, p in enumerate(pos, start=1):
        assert abs(p - (0.5 + j / 8 * (delta - 0.5))) < 1e-12
    for j, p in enumerate(reversed(neg), start=1):
        assert abs((1 - p) - (0.5 + j / 7 * (delta - 0.5))) < 1e-12


def _block_mse(W, levels):
    blocks = W.reshape(-1, 64).astype(np.float64)
    c = np.abs(blocks).max(axis=1, keepdims=True)
    x = blocks / c
    lv = np.asarray(levels, dtype=np.float64)
    idx = np.abs(x[:, :, None] - lv[None, None, :]).argmin(axis=2)
    return float(np.mean((lv[idx] * c - blocks) ** 2))     # error in weight units


def test_nf4_beats_uniform_grids_on_gaussian_blocks():
    W = np.random.default_rng(0).standard_normal((20000, 64)).astype(np.float32)
    mse_nf4 = _block_mse(W, nf4.nf4_levels())
    mse_u16 = _block_mse(W, np.linspace(-1.0, 1.0, 16))
    mse_i4 = _block_mse(W, np.arange(-7, 8) / 7.0)
    assert mse_nf4 < mse_u16 < mse_i4
    # N(0,1) weights: the NF4 error is below 1% of the weight variance
    assert mse_nf4 < 1e-2

"""Pins of the oracle's fp16 compute form (reading R11 of ``oracle/nf4.py``).

The binary16 rounding is written from the IEEE 754 definition; it is pinned
here by facts of that format (largest finite value, overflow threshold,
subnormal spacing, ties to even), by numpy's own float32 -> float16
conversion (an implementation the oracle does not call) over a wide sample,
and by the bit layout of known values. The fp16 dequantization is pinned to
the bf16 one, which the worked example and the encoder pins already fix: both
round the same fp32 product, so they may differ by at most half a bf16 step
plus half an fp16 step of that product, which a wrong code, block scale or
index would break.
"""

import numpy as np
import pytest

from oracle import linear as olin
from oracle import nf4 as onf4


@pytest.mark.parametrize("x,want", [
    (1.0, 1.0), (-2.5, -2.5), (65504.0, 65504.0),
    (65519.996, 65504.0),                 # below the overflow threshold
    (65520.0, np.inf), (-65520.0, -np.inf), (1e6, np.inf),
    (2.0 ** -24, 2.0 ** -24),             # smallest subnormal
    (2.0 ** -25, 0.0),                    # tie between 0 and 2^-24: even is 0
    (3 * 2.0 ** -25, 2.0 ** -23),         # tie between 1 and 2 steps: even is 2
    (2.0 ** -14, 2.0 ** -14),             # smallest normal
    (1 + 2.0 ** -11, 1.0),                # tie, keeps the even 1.0
    (1 + 3 * 2.0 ** -11, 1 + 2.0 ** -9),  # tie, goes up to the even neighbour
    (1 + 2.0 ** -11 + 2.0 ** -20, 1 + 2.0 ** -10),
    (2049.0, 2048.0), (2051.0, 2052.0),   # spacing 2 in [2048, 4096)
    (0.1, 0.0999755859375),
])
def test_fp16_round_ieee_facts(x, want):
    got = onf4.fp16_round(np.float32(x))
    assert got == want or (np.isinf(want) and got == want)


def test_fp16_round_keeps_signed_zero():
    z = onf4.fp16_round(np.array([-0.0, 0.0, -(2.0 ** -26)], dtype=np.float32))
    assert list(np.signbit(z)) == [True, False, True] and np.all(z == 0)


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (np.inf, 0x7C00), (-np.inf, 0xFC00),
    (2.0 ** -24, 0x0001), (2.0 ** -14, 0x0400), (0.5, 0x3800), (-0.0, 0x8000), (1 + 2.0 ** -10, 0x3C01),
])
def test_fp16_bit_layout(x, bits):
    assert int(onf4.fp16_bits_of(np.array([x]))[0]) == bits


def test_fp16_round_matches_numpy_conversion():
    rng = np.random.default_rng(1601)
    u = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    # bias the sample toward the interesting range: subnormals, ties, near-overflow
    e = rng.integers(-30, 17, size=200_000)
    y = (np.ldexp(rng.integers(2048, 4096, size=e.size) + rng.choice([0.0, 0.5, 0.25], size=e.size), e - 11)
         * rng.choice([-1.0, 1.0], size=e.size)).astype(np.float32)
    x = np.concatenate([x, y])
    ours = onf4.fp16_bits_of(onf4.fp16_round(x))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp16_dequant_brackets_bf16_dequant():
    rng = np.random.default_rng(1602)
    W = (rng.standard_normal((40, 512)) * 0.02).astype(np.float32)
    W[3, 64:128] = 0.0
    W[7, :64] *= 300.0                     # a block far from the others
    ow = onf4.NF4Weight(W)
    p = onf4.scaled_levels(ow.codes, ow.cprime, ow.levels).astype(np.float64)
    w16 = ow.dequant_f16()
    wb = ow.dequant().astype(np.float64)
    _, ex = np.frexp(np.abs(p))
    half16 = np.ldexp(1.0, np.maximum(ex - 1, -14) - 11)
    half_bf = np.ldexp(1.0, ex - 1 - 8)
    assert np.all(np.abs(w16 - wb) <= half16 + half_bf)
    assert np.all(np.abs(w16 - p) <= half16)
    # the bit patterns decode back to the same values
    dec = ow.dequant_f16_bits().view(np.float16).astype(np.float64)
    assert np.array_equal(dec, w16)
    assert np.all(w16[3, 64:128] == 0.0)


def test_fp16_floor_is_the_rounding_error():
    z = np.array([[1.0, 1 + 2.0 ** -12, 3.0]])
    want = np.linalg.norm([0.0, 2.0 ** -12, 0.0]) / np.linalg.norm(z)
    assert olin.fp16_floor(z) == pytest.approx(want, rel=1e-12)

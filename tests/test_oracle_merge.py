"""Pins for the oracle's adapter merge and unmerge (no GPU).

Pages: the trained adapter is folded into a dequantized copy of the base, not
into the 4-bit codes ("QLoRA: Quantized Low-Rank Adaptation", the two prices,
price 2; "QLoRA vs LoRA ...", converting back to full precision; "QLoRA
Explained ...", "Step 5: Save and Merge Adapters").

Each pin checks the oracle against something other than its own formula:
brute force over the bf16 grid for its rounding, a hand-worked example, the
pinned forward oracle (the merged layer must compute what the trained one
computes), exact integer round trips and the adapter-free special case.
"""

import numpy as np

from oracle import linear, merge


def _all_positive_bf16():
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint32)  # normal, finite
    return (bits << 16).view(np.float32).astype(np.float64)


def test_round_bf16_is_nearest_ties_to_even_by_brute_force():
    grid = _all_positive_bf16()
    g = np.random.default_rng(3)
    # random values, exact midpoints and grid points, both signs
    x = np.concatenate([g.uniform(1e-30, 1e30, 4000) * np.exp(g.uniform(-60, 60, 4000)),
                        (grid[100:-100:97] + grid[101:-99:97]) / 2, grid[::1013]])
    x = x[(x > grid[0]) & (x < grid[-1])]
    for sign in (1.0, -1.0):
        got = merge.round_bf16(sign * x)
        i = np.searchsorted(grid, x)  # grid[i-1] < x <= grid[i]
        lo, hi = grid[i - 1], grid[i]
        d_lo, d_hi = x - lo, hi - x
        lo_bits = (lo.astype(np.float32).view(np.uint32) >> 16)
        want = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo_bits % 2 == 0, lo, hi)))
        want = np.where(x == hi, hi, want)
        assert np.array_equal(got, sign * want)


def test_hand_worked_merge():
    # W' = [[1, -2], [0.5, 3]], A = [[1, 2]] (r = 1), B = [[0.5], [-1]], s = 2:
    # s B A = [[1, 2], [-2, -4]]  ->  merged = [[2, 0], [-1.5, -1]]
    Wd = np.array([[1.0, -2.0], [0.5, 3.0]])
    A = np.array([[1.0, 2.0]])
    B = np.array([[0.5], [-1.0]])
    for out in ("bf16", "fp32"):
        assert np.array_equal(merge.adapter_merge(Wd, A, B, 2.0, out), [[2.0, 0.0], [-1.5, -1.0]])
    # a value between two bf16 numbers: 1 + 2^-9 rounds to 1 in bf16, stays in fp32
    A1 = np.array([[2.0 ** -10, 0.0]])
    B1 = np.array([[1.0], [0.0]])
    assert merge.adapter_merge(Wd, A1, B1, 2.0, "bf16")[0, 0] == 1.0
    assert merge.adapter_merge(Wd, A1, B1, 2.0, "fp32")[0, 0] == 1.0 + 2.0 ** -9


def test_merged_layer_computes_the_trained_layer():
    g = np.random.default_rng(7)
    m, n, k, r, s = 12, 40, 128, 8, 0.25
    X = g.standard_normal((m, k))
    Wd = merge.round_bf16(g.standard_normal((n, k)) * 0.02)
    A = merge.round_bf16(g.uniform(-1, 1, (r, k)) / np.sqrt(k))
    B = merge.round_bf16(g.standard_normal((n, r)) * 0.01)
    Y, _ = linear.linear_fwd(X, Wd, A, B, s)          # the pinned forward oracle
    Yexact = X @ merge.merge_exact(Wd, A, B, s).T
    assert np.allclose(Yexact, Y, rtol=1e-12, atol=1e-13)
    # rounding the merged weight to bf16 moves each weight by at most half a bf16 ulp (2^-9 relative)
    Wm = merge.adapter_merge(Wd, A, B, s, "bf16")
    bound = np.abs(X) @ (np.abs(merge.merge_exact(Wd, A, B, s)) * 2.0 ** -9).T
    assert np.all(np.abs(X @ Wm.T - Y) <= bound + 1e-15)


def test_adapter_free_merge_is_the_dequantized_weight():
    g = np.random.default_rng(11)
    Wd = merge.round_bf16(g.standard_normal((16, 64)) * 0.02)
    A = np.zeros((4, 64))
    B = merge.round_bf16(g.standard_normal((16, 4)))
    for out in ("bf16", "fp32"):
        assert np.array_equal(merge.adapter_merge(Wd, A, B, 3.0, out), Wd)
        A2 = merge.round_bf16(g.standard_normal((4, 64)))
        assert np.array_equal(merge.adapter_merge(Wd, A2, np.zeros((16, 4)), 3.0, out), Wd)


def test_integer_round_trip_is_exact():
    g = np.random.default_rng(5)
    Wd = g.integers(-8, 9, (24, 64)).astype(np.float64)
    A = g.integers(-3, 4, (5, 64)).astype(np.float64)
    B = g.integers(-3, 4, (24, 5)).astype(np.float64)
    s = 2.0
    # every merged value is an integer of magnitude < 256: exact in bf16
    want = Wd + s * np.einsum("ij,jc->ic", B, A)
    assert np.abs(want).max() < 256
    Wm = merge.adapter_merge(Wd, A, B, s, "bf16")
    assert np.array_equal(Wm, want)
    assert np.array_equal(merge.adapter_unmerge(Wm, A, B, s), Wd)
    assert np.array_equal(merge.bf16_value_bits(Wm).view(np.uint16).astype(np.uint32) << 16,
                          Wm.astype(np.float32).view(np.uint32))

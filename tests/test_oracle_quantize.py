"""Pins for the oracle's first-level NF4 quantizer (no GPU).

Pages: 64-weight blocks scaled by their largest magnitude, each weight stored
as the nearest of the 16 levels, half a byte per weight ("QLoRA: Quantized
Low-Rank Adaptation": three-piece summary, the worked 8-weight block, and
"NF4: a 4-bit format matched to weight statistics").
"""

import json
import os
from fractions import Fraction

import numpy as np

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_codes(W, levels):
    """Exact rational argmin_j |w/c - L_j|, ties to the lower index; c = 0 -> 7."""
    lv = [Fraction(float(v)) for v in levels]
    out = np.zeros(W.shape, dtype=np.uint8)
    flat = W.reshape(-1, 64)
    for b, blk in enumerate(flat):
        c = max(Fraction(float(abs(v))) for v in blk)
        for i, w in enumerate(blk):
            if c == 0:
                code = 7
            else:
                x = Fraction(float(w)) / c
                dists = [abs(x - l) for l in lv]
                code = min(range(16), key=lambda j: (dists[j], j))
            out.reshape(-1, 64)[b, i] = code
    return out


def test_worked_example_from_the_page():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    w8 = np.array(g["weights"], dtype=np.float32)
    L = nf4.nf4_levels()
    # the page runs the example as one block; the format needs 64 weights per
    # block, so pad with zeros: padding changes neither the absmax nor the codes
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, :8] = w8
    assert nf4.block_absmax(W)[0] == np.float32(g["absmax"])
    codes = nf4.nf4_codes(W, L)
    assert np.array_equal(codes, _brute_codes(W, L))
    assert np.all(codes[0, 8:] == 7)
    assert len(L) == g["levels"]
    # storage of the 8 weights: 2 B each in bf16, half a byte each as codes
    assert w8.size * 2 == g["bf16_bytes"]
    assert nf4.pack_nibbles(codes[:, :8]).nbytes == g["nf4_bytes"]
    # the largest weight is reproduced exactly by its level and scale
    assert codes[0, 4] == 15 and L[codes[0, 4]] * g["absmax"] == 1.0
    # every reconstruction is the nearest level (brute force agrees), and the
    # error is below half the widest gap between levels
    rec = L[codes[0, :8]].astype(np.float64) * g["absmax"]
    assert np.max(np.abs(rec - w8)) <= np.max(np.diff(L.astype(np.float64))) / 2


def test_brute_force_random_tiny():
    rng = np.random.default_rng(1)
    L = nf4.nf4_levels()
    for scale in (1.0, 0.02, 3e-5, 7.0):
        W = (rng.standard_normal((3, 128)) * scale).astype(np.float32)
        assert np.array_equal(nf4.nf4_codes(W, L), _brute_codes(W, L))


def test_exact_ties_go_to_the_lower_level_and_neighbours_split():
    """A weight exactly on a midpoint between two levels takes the lower one;
    its fp32 neighbours split. Exact ties exist only where mu_j * c_b is an
    fp32 number; try two scales, c = 1 and c = 3 * 2^-7."""
    L = nf4.nf4_levels()
    L64 = L.astype(np.float64)
    mids = (L64[:-1] + L64[1:]) / 2
    total = 0
    for c in (1.0, 3.0 * 2.0 ** -7):
        ties = [(j, m * c) for j, m in enumerate(mids) if float(np.float32(m * c)) == m * c]
        W = np.zeros((1, 64), dtype=np.float32)
        W[0, 0] = np.float32(c)      # the block's absmax
        expect = {}
        for t, (j, w) in enumerate(ties):
            w32 = np.float32(w)
            W[0, 1 + 3 * t] = w32
            W[0, 2 + 3 * t] = np.nextafter(w32, np.float32(np.inf))
            W[0, 3 + 3 * t] = np.nextafter(w32, np.float32(-np.inf))
            expect[1 + 3 * t], expect[2 + 3 * t], expect[3 + 3 * t] = j, j + 1, j
        codes = nf4.nf4_codes(W, L)
        assert np.array_equal(codes, _brute_codes(W, L))
        for pos, code in expect.items():
            assert codes[0, pos] == code
        total += len(ties)
    assert total >= 4


def test_structural_invariants():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    W[3, 64:128] = 0.0                              # an all-zero block
    W[5, 7] = 0.0                                   # an isolated zero
    L = nf4.nf4_levels()
    codes = nf4.nf4_codes(W, L)
    assert codes.max() <= 15
    assert np.all(codes[3, 64:128] == 7)
    assert codes[5, 7] == 7
    blocks = W.reshape(-1, 64)
    cb = codes.reshape(-1, 64)
    for b in range(blocks.shape[0]):
        if not np.any(blocks[b]):
            continue
        i = int(np.argmax(np.abs(blocks[b])))
        assert cb[b, i] == (15 if blocks[b, i] > 0 else 0)
    # a power-of-two rescale of the tensor leaves every code unchanged
    assert np.array_equal(nf4.nf4_codes(W * np.float32(8.0), L), codes)
    assert np.array_equal(nf4.nf4_codes(W * np.float32(2.0 ** -20), L), codes)
    # a sign flip mirrors codes only where the levels are symmetric: at least
    # the block maxima map 15 <-> 0
    neg = nf4.nf4_codes(-W, L).reshape(-1, 64)
    for b in range(blocks.shape[0]):
        if np.any(blocks[b]):
            i = int(np.argmax(np.abs(blocks[b])))
            assert {int(cb[b, i]), int(neg[b, i])} == {0, 15}


def test_blocks_follow_rows_and_never_mix():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((4, 192)) * 0.02).astype(np.float32)
    W[2, 70] = 5.0           # outlier in block (row 2, block 1)
    c = nf4.block_absmax(W)
    assert c.shape == (12,)
    assert c[2 * 3 + 1] == np.float32(5.0)
    assert np.all(np.delete(c, 7) < 1.0)
    codes = nf4.nf4_codes(W, nf4.nf4_levels())
    # codes of the other blocks are unaffected by the outlier
    W2 = W.copy()
    W2[2, 70] = 0.0
    codes2 = nf4.nf4_codes(W2, nf4.nf4_levels())
    mask = np.ones((4, 192), dtype=bool)
    mask[2, 64:128] = False
    assert np.array_equal(codes[mask], codes2[mask])


def test_pack_nibble_order_and_round_trip():
    codes = np.array([[1, 2, 15, 0, 7, 8]], dtype=np.uint8)
    packed = nf4.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x0F, 0x87]]
    rng = np.random.default_rng(4)
    c = rng.integers(0, 16, size=(5, 128), dtype=np.uint8)
    assert np.array_equal(nf4.unpack_nibbles(nf4.pack_nibbles(c)), c)
    assert nf4.pack_nibbles(c).nbytes * 2 == c.size

"""Pins for the oracle's ablation variants (no GPU): the uniform INT4 grid
and the encoding without double quantization.

Pages: a uniform INT4 grid spaces its 16 values evenly while NF4 puts them
where a bell curve is dense, so NF4 reconstructs Gaussian blocks with less
error ("QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
"NF4: a 4-bit format matched to weight statistics"); double quantization
saves about 0.37 bit per parameter over fp32 block constants ("QLoRA
Explained ..." (gamut.so), "Double Quantization").
"""

import json
import os

import numpy as np

from oracle import nf4

from test_oracle_quantize import _brute_codes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_uniform_grid_shape():
    L = nf4.uniform4_levels().astype(np.float64)
    assert L.shape == (16,) and np.all(np.diff(L) > 0)
    assert L[0] == -1.0 and L[7] == 0.0 and L[14] == 1.0
    # symmetric about the zero level, evenly spaced to within fp32 rounding
    assert np.array_equal(L[:7], -L[14:7:-1])
    step = np.diff(L)
    assert np.max(np.abs(step - step.mean())) <= 2.0 ** -23
    assert abs(7.0 * L[8] - 1.0) <= 2.0 ** -23


def test_uniform_codes_match_brute_force_and_never_use_the_top_level():
    rng = np.random.default_rng(4)
    L = nf4.uniform4_levels()
    for scale in (1.0, 0.02, 3e-5):
        W = (rng.standard_normal((3, 128)) * scale).astype(np.float32)
        W[1, 64] = np.abs(W[1, 64:128]).max() * np.float32(1.0)   # a positive block maximum
        codes = nf4.nf4_codes(W, L)
        assert np.array_equal(codes, _brute_codes(W, L))
        assert codes.max() <= 14


def test_nf4_has_less_error_than_uniform_on_gaussian_blocks():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    errs = {}
    for name, L in (("nf4", nf4.nf4_levels()), ("int4", nf4.uniform4_levels())):
        o = nf4.NF4Weight(W, L, double_quant=False)
        c = o.absmax.astype(np.float64).reshape(-1, 1)
        rec = (L.astype(np.float64)[o.codes].reshape(-1, 64) * c).reshape(W.shape)
        errs[name] = np.mean((rec - W) ** 2)
        if name == "int4":
            # an even grid of step c/7 leaves errors spread evenly over
            # +-step/2 (variance step^2 / 12), except the block maximum, which
            # is exact: 63/64 of mean(c^2) / 588
            pred = 63.0 / 64.0 * np.mean(c ** 2) / 588.0
            assert abs(errs[name] / pred - 1.0) < 0.02
    assert errs["nf4"] < 0.8 * errs["int4"]


def test_without_double_quant_the_scale_is_the_block_absmax():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, :8] = np.array(g["weights"], dtype=np.float32)
    for L in (nf4.nf4_levels(), nf4.uniform4_levels()):
        o = nf4.NF4Weight(W, L, double_quant=False)
        assert o.code8 is None and o.mean is None
        assert o.cprime[0] == np.float32(g["absmax"])
        # with scale 1.0 every weight comes back as its level, rounded to bf16
        want = nf4.bf16_bits(L[o.codes[0]].astype(np.float32))
        assert np.array_equal(o.dequant_bits()[0], want)
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((8, 512)) * 0.02).astype(np.float32)
    o = nf4.NF4Weight(W, double_quant=False)
    assert np.array_equal(o.cprime, np.abs(W.reshape(-1, 64)).max(axis=1))
    # same codes as with double quantization: the codes use the exact absmax
    assert np.array_equal(o.codes, nf4.NF4Weight(W).codes)


def test_storage_without_double_quant():
    g = json.load(open(os.path.join(GOLDEN, "storage_closed_forms.json")))
    n, k = 4096, 4096
    nb = n * k // 64
    assert nf4.packed_bytes(n, k, double_quant=False) == n * k // 2 + 4 * nb
    bits_nodq = 8.0 * nf4.packed_bytes(n, k, double_quant=False) / (n * k)
    bits_dq = 8.0 * nf4.packed_bytes(n, k) / (n * k)
    assert bits_nodq == 4.5
    # the difference is the page's saving of about 0.37 bit per parameter
    assert abs((bits_nodq - bits_dq) - g["dq_saving_bits_per_param_about"]) < 0.01


# --------------------------------------------------------------------------- bf16 block scale (no double quant)
#
# "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev): the worked
# 8-weight block stores its scale (the largest magnitude) in BF16, and the
# 65B arithmetic after it counts one BF16 scalar per 64-weight block.

from fractions import Fraction  # noqa: E402


def _brute_codes_against(W, levels, scales):
    """Exact rational nearest level to w / c for a given per-block c (ties to
    the lower index; c = 0 -> code 7)."""
    lv = [Fraction(float(v)) for v in levels]
    out = np.zeros(W.shape, dtype=np.uint8)
    flat = W.reshape(-1, 64)
    for b, blk in enumerate(flat):
        c = Fraction(float(scales[b]))
        for i, w in enumerate(blk):
            if c == 0:
                code = 7
            else:
                x = Fraction(float(w)) / c
                code = min(range(16), key=lambda j: (abs(x - lv[j]), j))
            out.reshape(-1, 64)[b, i] = code
    return out


def _torch_bf16(x):
    import torch
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_bf16_scale_storage_is_4_25_bits_and_the_pages_35_gb():
    g = json.load(open(os.path.join(GOLDEN, "storage_closed_forms.json")))
    n, k = 8192, 8192
    assert nf4.packed_bytes(n, k, double_quant=False, scale_bits=16) == n * k // 2 + 2 * (n * k // 64)
    assert 8.0 * nf4.packed_bytes(n, k, double_quant=False, scale_bits=16) / (n * k) == 4.25
    assert nf4.bits_per_weight(double_quant=False, scale_bits=16) == 4.25
    # 65B parameters at 4.25 bit: the page's "about 35 GB" (4.5 bit would be 36.6)
    gb = g["params"] * 4.25 / 8 / 1e9
    assert abs(gb - g["nf4_with_scales_GB_about"]) < 0.6
    assert abs(g["params"] * 4.5 / 8 / 1e9 - g["nf4_with_scales_GB_about"]) > 1.5


def test_bf16_scale_worked_block():
    """The page's block: scale 1.00 in BF16 (bit pattern 0x3F80), every
    weight snapped to its nearest level."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, :8] = np.array(g["weights"], dtype=np.float32)
    o = nf4.NF4Weight(W, double_quant=False, scale_dtype="bf16")
    assert o.code8 is None and o.mean is None
    assert o.s2.dtype == np.uint16 and int(o.s2[0]) == 0x3F80 and o.cprime[0] == np.float32(g["absmax"])
    assert np.array_equal(o.codes, _brute_codes_against(W, nf4.nf4_levels(), [1.0]))


def test_bf16_scale_codes_brute_force_with_fp32_weights():
    """fp32 weights whose block absmax is not a bf16 number: the stored scale
    is torch's bf16 rounding of it (above or below), and the codes are the
    exact nearest levels against that stored scale, end levels included for
    weights beyond it."""
    rng = np.random.default_rng(21)
    for L in (nf4.nf4_levels(), nf4.uniform4_levels()):
        W = (rng.standard_normal((4, 192)) * 0.02).astype(np.float32)
        W[0, 10] = np.float32(0.0501)           # absmax rounds down in bf16
        W[1, 70] = np.float32(-0.0507)          # absmax rounds up in bf16
        W[2, 128:192] = 0.0                     # an all-zero block
        o = nf4.NF4Weight(W, L, double_quant=False, scale_dtype="bf16")
        absmax = np.abs(W.reshape(-1, 64)).max(axis=1)
        want_c = _torch_bf16(absmax)
        assert np.array_equal(o.cprime.view(np.uint32), want_c.view(np.uint32))
        assert np.array_equal(o.s2, (want_c.view(np.uint32) >> 16).astype(np.uint16))
        assert np.any(want_c < absmax) and np.any(want_c > absmax)
        assert np.array_equal(o.codes, _brute_codes_against(W, L, want_c))
        # dequant = RN_bf16(L[code] * c') with c' the stored bf16 scale
        prod = (L[o.codes].reshape(-1, 64) * want_c[:, None]).astype(np.float32).reshape(W.shape)
        assert np.array_equal(o.dequant_bits(), nf4.bf16_bits(prod))


def test_bf16_scale_is_lossless_for_bf16_weights():
    """bf16 weights: the absmax is a bf16 number, so the 4.25-bit form has the
    fp32 form's scales and codes exactly."""
    rng = np.random.default_rng(22)
    W = _torch_bf16(rng.standard_normal((16, 512)) * 0.02)
    a = nf4.NF4Weight(W, double_quant=False, scale_dtype="bf16")
    b = nf4.NF4Weight(W, double_quant=False)
    assert np.array_equal(a.codes, b.codes)
    assert np.array_equal(a.cprime.view(np.uint32), b.cprime.view(np.uint32))
    assert np.array_equal(a.dequant_bits(), b.dequant_bits())

"""Pins for the oracle's double quantization, dequantization and storage
arithmetic (no GPU).

Pages: the block constants are themselves quantized to 8-bit floating point,
saving about 0.37 bit per parameter, roughly 3 GB at 65B ("QLoRA Explained
...", "Double Quantization"); the 65B base is 130 GB in bf16 and 32.5 GB as
half-byte codes, about 35 GB with its scales ("QLoRA: Quantized Low-Rank
Adaptation", the storage arithmetic after the worked block); blocks are
expanded back to bf16 right before the multiply (same page, three-piece
summary).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- E4M3 table

def test_e4m3_table_matches_torch_float8_decoding():
    vals, pats = nf4.e4m3_table()
    assert vals.size == 253 and np.all(np.diff(vals) > 0)
    assert vals[0] == -448.0 and vals[-1] == 448.0 and 0.0 in vals
    allbits = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        mine = nf4.e4m3_decode(b)
        if math.isnan(mine):
            assert math.isnan(allbits[b])
        else:
            assert mine == allbits[b], b
    # every stored pattern decodes to its table value
    for v, p in zip(vals, pats):
        assert allbits[p] == v


def _e4m3_nearest_brute(x: Fraction) -> float:
    vals, _ = nf4.e4m3_table()
    fv = [Fraction(float(v)) for v in vals]
    return float(fv[min(range(len(fv)), key=lambda i: (abs(x - fv[i]), i))])


def test_e4m3_nearest_agrees_with_brute_force_and_torch_rounding():
    rng = np.random.default_rng(5)
    c = np.abs(rng.standard_normal(1024) * 0.05).astype(np.float32)
    code8, s2, mean = nf4.double_quantize(c)
    vals = np.array([nf4.e4m3_decode(int(b)) for b in code8])
    d = (c - mean).astype(np.float32)
    s = s2[np.arange(c.size) // 256]
    for i in range(0, c.size, 7):
        x = Fraction(float(d[i])) / Fraction(float(s[i]))
        assert vals[i] == _e4m3_nearest_brute(x)
    # away from exact ties, torch's round-to-nearest-even conversion agrees
    ratio = (d.astype(np.float64) / s.astype(np.float64))
    t = torch.from_numpy(ratio).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(t, vals)


def test_e4m3_ties_go_to_the_lower_value():
    """Build one chunk whose mean is exactly 1 and whose s2 is exactly 2^-10,
    so d / s2 lands exactly on E4M3 midpoints and on their fp32 neighbours."""
    vals, _ = nf4.e4m3_table()
    e = 2.0 ** -10
    mid = (vals[200] + vals[201]) / 2
    above = float(np.nextafter(np.float32(1.0 + mid * e), np.float32(2.0))) - 1.0
    devs = [448.0 * e, mid * e, above]
    devs = devs + [-v for v in devs]                   # deviations sum to zero
    c = np.array([1.0 + v for v in devs] + [1.0] * (256 - len(devs)), dtype=np.float32)
    assert all(float(x) - 1.0 == v for x, v in zip(c, devs))
    code8, s2, mean = nf4.double_quantize(c)
    assert mean == np.float32(1.0) and s2[0] == np.float32(e)
    got = [nf4.e4m3_decode(int(b)) for b in code8[:6]]
    assert got[0] == 448.0 and got[3] == -448.0
    assert got[1] == vals[200]            # +mid: tie between vals[200] and vals[201] -> lower
    assert got[4] == -vals[201]           # -mid: tie between -vals[201] and -vals[200] -> lower
    assert got[2] == vals[201]            # just above +mid -> upper
    assert got[5] == -vals[201]           # just below -mid -> lower
    for i in range(6):
        assert got[i] == _e4m3_nearest_brute(Fraction(float(c[i]) - 1.0) / Fraction(e))


# ------------------------------------------------------------- second level

def test_mean_is_fixed_order_and_close_to_exact():
    rng = np.random.default_rng(6)
    for nb in (1, 255, 256, 257, 4096, 3000):
        c = np.abs(rng.standard_normal(nb)).astype(np.float32)
        m = nf4.dq_mean(c)
        exact = math.fsum(float(v) for v in c) / nb
        assert abs(float(m) - exact) <= float(np.spacing(np.float32(exact)))
        # the order is sequential per 256-run, then across runs
        total = 0.0
        for j in range(0, nb, 256):
            run = 0.0
            for v in c[j:j + 256]:
                run += float(v)
            total += run
        assert m == np.float32(total / nb)


def test_chunk_extremes_map_to_448_and_decode_error_is_bounded():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((512, 512)) * 0.02).astype(np.float32)
    c = nf4.block_absmax(W)
    code8, s2, mean = nf4.double_quantize(c)
    assert s2.size == c.size // 256
    d = (c - mean).astype(np.float32)
    vals, _ = nf4.e4m3_table()
    gaps = np.diff(vals)
    fp8 = np.array([nf4.e4m3_decode(int(b)) for b in code8])
    for j in range(s2.size):
        dj = d[j * 256:(j + 1) * 256]
        i = int(np.argmax(np.abs(dj)))
        assert abs(fp8[j * 256 + i]) == 448.0
        assert s2[j] == np.float32(np.abs(dj).max()) / np.float32(448.0)
    # |d/s2 - fp8| is at most half the local gap of the E4M3 grid
    ratio = d.astype(np.float64) / s2[np.arange(c.size) // 256].astype(np.float64)
    idx = np.searchsorted(vals, fp8)
    lo_gap = np.where(idx > 0, gaps[np.maximum(idx - 1, 0)], np.inf)
    hi_gap = np.where(idx < gaps.size, gaps[np.minimum(idx, gaps.size - 1)], np.inf)
    assert np.all(np.abs(ratio - fp8) <= np.maximum(lo_gap, hi_gap) / 2 + 1e-12)
    # reconstructed scales: relative error a few percent at most
    cp = nf4.decode_scales(code8, s2, mean)
    rel = np.abs(cp.astype(np.float64) - c) / c
    assert np.sqrt(np.mean(rel ** 2)) < 0.01 and rel.max() < 0.05


def test_single_block_and_zero_chunk_special_cases():
    # one block: d = 0 -> s2 = 0 -> code 0x00 -> c' = mean = c exactly
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, :8] = [0.90, -0.45, 0.15, -0.30, 1.00, -0.10, 0.25, -0.60]
    q = nf4.NF4Weight(W)
    assert q.s2.tolist() == [0.0] and q.code8.tolist() == [0]
    assert q.cprime[0] == q.absmax[0] == np.float32(1.0)
    # a chunk of identical scales is a zero chunk too
    c = np.full(512, 0.125, dtype=np.float32)
    code8, s2, mean = nf4.double_quantize(c)
    assert mean == np.float32(0.125) and np.all(s2 == 0) and np.all(code8 == 0)
    assert np.all(nf4.decode_scales(code8, s2, mean) == np.float32(0.125))


def test_scale_decode_is_two_separate_roundings():
    # fp8 value 1.125 (0x39), s2 and mean chosen so a fused multiply-add would
    # round differently from RN(RN(a*b)+c)
    s2 = np.array([np.float32(1.0) + np.float32(2.0 ** -23)], dtype=np.float32)
    a = np.float32(nf4.e4m3_decode(0x39))
    prod = np.float32(a * s2[0])
    mean = np.float32(-float(prod))
    code8 = np.array([0x39], dtype=np.uint8)
    cp = nf4.decode_scales(code8, s2, mean)[0]
    assert cp == np.float32(0.0)                          # separately rounded: cancels exactly
    fused = float(Fraction(float(a)) * Fraction(float(s2[0])) + Fraction(float(mean)))
    assert fused != 0.0                                   # a fused version would not


# ------------------------------------------------------------------ bf16

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    # add exact ties (lower 16 bits = 0x8000) with both parities of the kept bit
    u = rng.integers(0, 2 ** 31, 2000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, np.array([0.0, -0.0], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.bf16_bits(x), ref)


def test_dequant_special_values_and_size():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    W[10, :64] = 0.0
    q = nf4.NF4Weight(W)
    Wd = q.dequant()
    assert Wd.shape == W.shape and Wd.dtype == np.float32
    assert np.all(Wd[10, :64] == 0.0)
    # the argmax of each block is reconstructed as +-RN_bf16(c')
    blocks = W.reshape(-1, 64)
    wd = Wd.reshape(-1, 64)
    cp_bf16 = nf4.bf16_bits_to_f32(nf4.bf16_bits(q.cprime))
    for b in range(blocks.shape[0]):
        if not np.any(blocks[b]):
            continue
        i = int(np.argmax(np.abs(blocks[b])))
        assert abs(wd[b, i]) == cp_bf16[b]
    # sanity: 4-bit storage is a coarse approximation (about 9% relative)
    rel = np.linalg.norm(Wd - W) / np.linalg.norm(W)
    assert 0.05 < rel < 0.15


def test_dequant_bits_are_bf16_of_fp32_products():
    rng = np.random.default_rng(10)
    codes = rng.integers(0, 16, size=(8, 128), dtype=np.uint8)
    cp = (np.abs(rng.standard_normal(16)) * 0.05).astype(np.float32)
    L = nf4.nf4_levels()
    got = nf4.dequant_bits(codes, cp, L)
    # independent route: torch multiplies in fp32 and converts with RNE
    prod = torch.from_numpy(L[codes]) * torch.from_numpy(np.repeat(cp.reshape(8, 2), 64, axis=1))
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# -------------------------------------------------------- storage closed forms

def test_storage_closed_forms_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "storage_closed_forms.json")))
    P = g["params"]
    assert P * 2 / 1e9 == g["bf16_GB"]
    # half a byte per weight of codes
    assert nf4.packed_bytes(1024, 1024) - (1024 * 1024 // 64 + 4 * 64 + 4) == 1024 * 1024 * g["nf4_bytes_per_weight"]
    assert P * g["nf4_bytes_per_weight"] / 1e9 == g["nf4_codes_GB"]
    # double quantization: 4.5 bits/weight with fp32 block constants, 4.127 with
    # 8-bit constants + one fp32 per 256 blocks; the saving is the pages' ~0.37
    without = nf4.bits_per_weight(double_quant=False, scale_bits=32)
    with_dq = nf4.bits_per_weight(double_quant=True)
    saving = without - with_dq
    assert without == 4.5 and abs(with_dq - 4.126953125) < 1e-12
    assert abs(saving - g["dq_saving_bits_per_param_about"]) < 0.005
    assert abs(P * saving / 8 / 1e9 - g["dq_saving_GB_about_65B"]) < 0.05
    # with its scales the 65B base is "about 35 GB": between codes-only and the
    # no-double-quant fp32 figure, and within 2 GB of 35
    total = P * with_dq / 8 / 1e9
    assert g["nf4_codes_GB"] < total < P * without / 8 / 1e9
    assert abs(total - g["nf4_with_scales_GB_about"]) < 2.0
    # exact packed size on a real shape equals the bit arithmetic
    n, k = 8192, 8192
    assert nf4.packed_bytes(n, k) * 8 == n * k * 4 + (n * k // 64) * 8 + (n * k // 64 // 256) * 32 + 32

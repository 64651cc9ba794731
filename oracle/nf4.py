"""NF4 storage format, plain CPU oracle (numpy, fp64 where a decision is made).

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may import this.

Sources (web pages on QLoRA; cited by title and section):

* [QX]  "QLoRA Explained: Fine-Tune 70B+ LLMs on a Single GPU" (gamut.so),
        sections "4-Bit NormalFloat (NF4) Quantization" and
        "Double Quantization".
* [QQ]  "QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev),
        the three-piece summary (storage / compute / learning), the worked
        8-weight block, the section "NF4: a 4-bit format matched to weight
        statistics" and the double-quantization paragraph after it.

What the pages fix, in my words:
  - a weight is stored as one of 16 levels (4 bits), two weights per byte;
  - the levels are quantiles of a normal distribution, rescaled so that the
    largest magnitude is 1;
  - each block of 64 consecutive weights has its own scale, the largest
    absolute value in the block, and a weight is stored as the level nearest
    to weight/scale;
  - the block scales are themselves quantized to 8-bit floating point in
    blocks ("double quantization"), which saves about 0.37 bit per weight;
  - right before a multiply, the 64-block is expanded back to bf16.

Readings where the pages leave a step open:
  R1 levels: 7 negative quantiles, an exact zero and 8 positive quantiles of
     N(0,1), taken at evenly spaced probabilities between 1/2 and delta on
     each side, delta = ((1-1/30) + (1-1/32))/2, divided by Phi^-1(delta),
     computed in fp64 and rounded once to fp32.
  R2 first-level scale c_b is fp32 (the 0.37-bit saving only works out for a
     32-bit constant).
  R3 8-bit format of the second level: OCP FP8 E4M3 (finite range +-448).
  R4 one fp32 mean per tensor is subtracted from the block scales before the
     8-bit step; 256 scales share one fp32 second-level scale s2.
  R5 nearest-level ties go to the lower index, for NF4 and for E4M3.
  R6 an all-zero 64-block stores code 7 (the zero level); a chunk whose
     centred scales are all zero stores s2 = 0 and code8 = 0x00.
  R7 dequant: c' = RN32(RN32(fp8(code8) * s2) + mean), two separately
     rounded fp32 operations; w' = RN_bf16(RN32(L[code] * c')), bf16 with
     round-to-nearest-even.
  R8 nibble order: element 2t goes in the low nibble of byte t.

Ablation variants the pages contrast NF4 and double quantization with
(QQ "NF4: a 4-bit format matched to weight statistics": a uniform INT4 grid
spends code points evenly; QX "Double Quantization": the saving over keeping
the block constants in full precision):
  R9  uniform INT4 grid: L_i = RN32((i - 7) / 7), i = 0..15 -- evenly spaced,
      -1 at index 0, the exact zero at index 7 (where R6 puts all-zero blocks),
      +1 at index 14; index 15 (8/7) lies beyond any block's largest
      magnitude and is never chosen (the symmetric absmax INT4 grid).
  R10 no double quantization: c' = c_b, the fp32 block absmax, stored as is
      (one fp32 per block instead of one byte plus shares of s2 and mean).
  R12 no double quantization with a bf16 block scale (QQ's worked block and
      its 65B arithmetic store "one BF16 scalar per 64-weight block"):
      c_b = RN_bf16(block absmax), stored as its bf16 bit pattern (16 bits per
      block: 4.25 bit per weight); the codes are the nearest levels to
      w / c_b for that stored c_b (the scale the dequant will use), so a
      weight above c_b in magnitude takes an end level; c' = c_b. A block
      whose c_b is zero stores code 7 (R6). For bf16 weights the absmax is
      already a bf16 number: c_b equals the fp32 form's scale and the codes
      are the same, at 0.25 bit per weight less storage.
  R11 fp16 compute (the other 16-bit compute type the pages use: "QLoRA vs
      LoRA ..." (instagit.com), "QLoRA Fine-Tuning with 4-Bit Quantization",
      a float16 compute dtype): w' = RN_fp16(RN32(L[code] * c')), IEEE
      binary16 with round-to-nearest-even, gradual underflow below 2^-14 and
      overflow to infinity from 65520 up.
"""

from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

BLOCK = 64        # weights per first-level block [QQ]
DQ_BLOCK = 256    # first-level scales per second-level block (reading R4)
E4M3_MAX = 448.0  # largest finite OCP E4M3 magnitude (reading R3)


# --------------------------------------------------------------------------
# Codebook  [QX "4-Bit NormalFloat (NF4) Quantization"; QQ "NF4: a 4-bit
# format matched to weight statistics"]
# --------------------------------------------------------------------------

def normal_quantile(p: float) -> float:
    """Phi^-1(p) of the standard normal, fp64 (the stdlib's inverse CDF)."""
    return NormalDist(0.0, 1.0).inv_cdf(p)


def nf4_delta() -> float:
    """Outermost probability delta of reading R1."""
    return 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


def nf4_levels_fp64() -> list[float]:
    """The 16 NF4 levels in fp64, ascending (reading R1).

    Eight positive levels sit at the normal quantiles of probabilities
    1/2 + (j/8)(delta - 1/2), j = 1..8; seven negative levels mirror the
    quantiles of 1/2 + (j/7)(delta - 1/2), j = 1..7; one level is exactly 0.
    All are divided by Phi^-1(delta) so the extreme levels are -1 and +1.
    """
    delta = nf4_delta()
    positive = [normal_quantile(0.5 + (j / 8.0) * (delta - 0.5)) for j in range(1, 9)]
    negative = [-normal_quantile(0.5 + (j / 7.0) * (delta - 0.5)) for j in range(1, 8)]
    top = normal_quantile(delta)
    return sorted(v / top for v in negative + [0.0] + positive)


def nf4_levels() -> np.ndarray:
    """The 16 NF4 levels rounded once to fp32 (index 0 = -1, 7 = 0, 15 = +1)."""
    return np.array(nf4_levels_fp64(), dtype=np.float64).astype(np.float32)


def uniform4_levels() -> np.ndarray:
    """The uniform INT4 grid of reading R9, each level rounded once to fp32
    (the rational (i - 7)/7 is rounded directly, not through fp64)."""
    from fractions import Fraction
    out = []
    for i in range(16):
        q = Fraction(i - 7, 7)
        lo = np.float32(float(q))                      # within one fp32 ulp of q
        cands = [np.nextafter(lo, np.float32(-2)), lo, np.nextafter(lo, np.float32(2))]
        best = min(cands, key=lambda v: (abs(Fraction(float(v)) - q),
                                         int(np.asarray(v, np.float32).view(np.uint32)) & 1))
        out.append(best)
    return np.array(out, dtype=np.float32)


# --------------------------------------------------------------------------
# First level: blockwise absmax + nearest level  [QQ worked 8-weight block and
# "NF4: a 4-bit format ..." paragraph on 64-weight absmax blocks]
# --------------------------------------------------------------------------

def block_absmax(W: np.ndarray) -> np.ndarray:
    """c_b = max |w| over each 64-block of the row-major flattening (fp32, exact)."""
    W = np.asarray(W, dtype=np.float32)
    assert W.ndim == 2 and W.shape[1] % BLOCK == 0, "K must be a multiple of 64"
    return np.abs(W.reshape(-1, BLOCK)).max(axis=1)


def nf4_codes(W: np.ndarray, levels: np.ndarray, rows_per_chunk: int = 256, scales=None) -> np.ndarray:
    """Unpacked 4-bit codes [N, K] (uint8), nearest level to w / c_b.

    Nearest with ties to the lower index (R5) is evaluated without dividing:
    code = #{ j in 0..14 : w > mu_j * c_b }, mu_j the midpoint of levels j and
    j+1. mu_j and mu_j * c_b are exact in fp64 (fp32 inputs), so every
    comparison is exact. A block with c_b = 0 (all-zero) gets code 7 (R6).
    c_b is the block absmax unless ``scales`` (one fp32 per block, R12)
    gives the scale the codes are taken against.
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    lv = levels.astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2.0                      # 15 midpoints
    codes = np.empty((N, K), dtype=np.uint8)
    bpr = K // BLOCK
    for r0 in range(0, N, rows_per_chunk):
        blk = W[r0:r0 + rows_per_chunk].astype(np.float64).reshape(-1, BLOCK)
        if scales is None:
            c = np.abs(blk).max(axis=1)
        else:
            r1 = min(r0 + rows_per_chunk, N)
            c = np.asarray(scales, dtype=np.float32)[r0 * bpr:r1 * bpr].astype(np.float64)
        thr = c[:, None] * mids[None, :]                 # [nb, 15]
        q = (blk[:, :, None] > thr[:, None, :]).sum(axis=2).astype(np.uint8)
        q[c == 0.0] = 7
        codes[r0:r0 + rows_per_chunk] = q.reshape(-1, K)
    return codes


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte, element 2t in the low nibble (R8). [N, K] -> [N, K/2]."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_nibbles``."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# OCP FP8 E4M3, written from the format's definition (reading R3)
# --------------------------------------------------------------------------

def e4m3_decode(bits: int) -> float:
    """Value of one E4M3 bit pattern: 1 sign, 4 exponent bits (bias 7),
    3 mantissa bits, subnormals at exponent 0, S.1111.111 is NaN, no infinity."""
    sign = -1.0 if bits & 0x80 else 1.0
    e = (bits >> 3) & 0xF
    m = bits & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> tuple[np.ndarray, np.ndarray]:
    """The 253 distinct finite E4M3 values ascending (one zero, -0 and NaN
    dropped) and the bit pattern that stores each."""
    entries = []
    for bits in range(256):
        v = e4m3_decode(bits)
        if math.isnan(v) or (v == 0.0 and bits & 0x80):
            continue
        entries.append((v, bits))
    entries.sort()
    vals = np.array([v for v, _ in entries], dtype=np.float64)
    pats = np.array([b for _, b in entries], dtype=np.uint8)
    return vals, pats


# --------------------------------------------------------------------------
# Second level: double quantization of the block constants
# [QX "Double Quantization"; QQ double-quantization paragraph]
# --------------------------------------------------------------------------

def dq_mean(c: np.ndarray) -> np.float32:
    """Tensor mean of the block scales in a fixed order (reading R4).

    Each run of 256 consecutive c_b is summed left to right in fp64; the run
    sums are then added left to right in fp64; the total is divided by nb in
    fp64 and rounded once to fp32. (``np.cumsum`` is a sequential running sum.)
    """
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    nb = c.size
    total = 0.0
    for j0 in range(0, nb, DQ_BLOCK):
        run = float(np.cumsum(c[j0:j0 + DQ_BLOCK])[-1])
        total = total + run
    return np.float32(total / float(nb))


def double_quantize(c: np.ndarray):
    """Quantize the fp32 block scales c_b [nb] to 8 bits.

    Returns (code8 uint8 [nb], s2 fp32 [ceil(nb/256)], mean fp32).
      d_b    = RN32(c_b - mean)
      s2_j   = RN32(max_{b in chunk j} |d_b| / 448)
      code8  = bit pattern of the E4M3 value nearest to d_b / s2_j (ties to the
               lower value), found as #{k : d_b > nu_k * s2_j} with nu_k the
               exact midpoints of the sorted table; s2_j = 0 gives 0x00.
    """
    c = np.asarray(c, dtype=np.float32)
    nb = c.size
    nc = -(-nb // DQ_BLOCK)
    mean = dq_mean(c)
    d = (c - mean).astype(np.float32)                   # one fp32 subtraction each
    vals, pats = e4m3_table()
    nu = (vals[:-1] + vals[1:]) / 2.0                   # 252 exact midpoints
    code8 = np.zeros(nb, dtype=np.uint8)
    s2 = np.zeros(nc, dtype=np.float32)
    for j in range(nc):
        dj = d[j * DQ_BLOCK:(j + 1) * DQ_BLOCK]
        a2 = np.abs(dj).max()
        s2j = np.float32(a2) / np.float32(E4M3_MAX)     # fp32 division, RN
        s2[j] = s2j
        if s2j == 0.0:
            continue
        thr = nu * float(s2j)                            # exact in fp64
        idx = (dj.astype(np.float64)[:, None] > thr[None, :]).sum(axis=1)
        code8[j * DQ_BLOCK:(j + 1) * DQ_BLOCK] = pats[idx]
    return code8, s2, mean


def decode_scales(code8: np.ndarray, s2: np.ndarray, mean) -> np.ndarray:
    """c'_b = RN32(RN32(fp8(code8_b) * s2_{b//256}) + mean), no fused multiply-add."""
    code8 = np.asarray(code8, dtype=np.uint8)
    fp8 = np.array([e4m3_decode(int(b)) for b in range(256)], dtype=np.float64).astype(np.float32)
    v = fp8[code8]
    s = np.asarray(s2, dtype=np.float32)[np.arange(code8.size) // DQ_BLOCK]
    prod = (v * s).astype(np.float32)                   # fp32 multiply, RN
    return (prod + np.float32(mean)).astype(np.float32)  # fp32 add, RN


# --------------------------------------------------------------------------
# bf16 and dequantization  [QQ three-piece summary, "compute: still 16 bits"]
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite input)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_odd = (u >> 16) & 1
    return ((u + 0x7FFF + keep_odd) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dequant_bits(codes: np.ndarray, cprime: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """w'_i = RN_bf16(RN32(L[code_i] * c'_b)) as bf16 bit patterns, [N, K] uint16."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    lv = np.asarray(levels, dtype=np.float32)
    c = np.asarray(cprime, dtype=np.float32).reshape(N, K // BLOCK)
    prod = (lv[codes].reshape(N, K // BLOCK, BLOCK) * c[:, :, None]).astype(np.float32)
    return bf16_bits(prod.reshape(N, K))


def dequant(codes, cprime, levels) -> np.ndarray:
    """Same as ``dequant_bits`` but as fp32 values holding the bf16 numbers."""
    return bf16_bits_to_f32(dequant_bits(codes, cprime, levels))


# --------------------------------------------------------------------------
# fp16 (reading R11), written from the IEEE 754 binary16 definition:
# 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; normal numbers
# 2^-14 <= |x| <= 65504, subnormal spacing 2^-24.
# --------------------------------------------------------------------------

FP16_MAX = 65504.0


def fp16_round(x) -> np.ndarray:
    """Round to the nearest binary16 value, ties to even, in fp64 (exact for
    fp32 input): the spacing at |x| in [2^e, 2^(e+1)) is 2^(e-10), and 2^-24
    throughout the subnormal range e < -14. Overflow gives +-inf (a rounded
    magnitude above 65504 is one that reached 65536)."""
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(np.abs(x))                  # |x| = m 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -14)                  # floor(log2 |x|), clamped at the subnormal range
    q = np.ldexp(1.0, e - 10)                    # spacing of binary16 at |x|
    r = np.rint(x / q) * q                       # rint: nearest integer, ties to even; x / q exact
    r = np.where(np.abs(r) > FP16_MAX, np.copysign(np.inf, x), r)
    return np.where(r == 0, np.copysign(0.0, x), r)


def fp16_bits_of(v) -> np.ndarray:
    """Bit patterns of values that are already binary16 numbers (fp64 in)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint16) << np.uint16(15)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.uint16)
    inf = np.isinf(a)
    sub = (a < 2.0 ** -14) & ~inf
    nrm = ~sub & ~inf
    out[sub] = (a[sub] / 2.0 ** -24).astype(np.uint16)
    m, ex = np.frexp(a[nrm])                     # a = m 2^ex, m in [0.5, 1)
    biased = (ex - 1 + 15).astype(np.uint16)
    frac = ((m * 2.0 - 1.0) * 1024.0).astype(np.uint16)
    out[nrm] = (biased << np.uint16(10)) | frac
    out[inf] = 0x7C00
    return out | sign


def scaled_levels(codes: np.ndarray, cprime: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """RN32(L[code_i] * c'_b), the fp32 product both 16-bit roundings start from, [N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    lv = np.asarray(levels, dtype=np.float32)
    c = np.asarray(cprime, dtype=np.float32).reshape(N, K // BLOCK)
    return (lv[codes].reshape(N, K // BLOCK, BLOCK) * c[:, :, None]).astype(np.float32).reshape(N, K)


def dequant_f16_bits(codes: np.ndarray, cprime: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """w'_i = RN_fp16(RN32(L[code_i] * c'_b)) as binary16 bit patterns, [N, K] uint16."""
    return fp16_bits_of(fp16_round(scaled_levels(codes, cprime, levels)))


# --------------------------------------------------------------------------
# Whole encode, and storage arithmetic
# --------------------------------------------------------------------------

class NF4Weight:
    """Everything the encoder produces for one [N, K] weight. ``levels``
    selects the 16-level grid (NF4 by default, R9 for the uniform ablation);
    ``double_quant=False`` keeps one scale per block instead (code8 and mean
    are then None): the fp32 block absmax in s2 (R10), or with
    ``scale_dtype="bf16"`` its bf16 rounding, s2 holding the uint16 bit
    patterns (R12)."""

    def __init__(self, W: np.ndarray, levels: np.ndarray | None = None, double_quant: bool = True,
                 scale_dtype: str = "fp32"):
        W = np.asarray(W, dtype=np.float32)
        assert scale_dtype in ("fp32", "bf16") and (scale_dtype == "fp32" or not double_quant)
        self.shape = W.shape
        self.scale_dtype = scale_dtype
        self.levels = nf4_levels() if levels is None else levels
        self.absmax = block_absmax(W)
        if scale_dtype == "bf16":
            self.s2 = bf16_bits(self.absmax)
            self.cprime = bf16_bits_to_f32(self.s2)
            self.codes = nf4_codes(W, self.levels, scales=self.cprime)
        else:
            self.codes = nf4_codes(W, self.levels)
        self.packed = pack_nibbles(self.codes)
        if double_quant:
            self.code8, self.s2, self.mean = double_quantize(self.absmax)
            self.cprime = decode_scales(self.code8, self.s2, self.mean)
        elif scale_dtype == "fp32":
            self.code8, self.mean = None, None
            self.s2 = self.absmax.astype(np.float32).copy()
            self.cprime = self.s2
        else:
            self.code8, self.mean = None, None

    def dequant_bits(self) -> np.ndarray:
        return dequant_bits(self.codes, self.cprime, self.levels)

    def dequant(self) -> np.ndarray:
        return dequant(self.codes, self.cprime, self.levels)

    def dequant_f16_bits(self) -> np.ndarray:
        return dequant_f16_bits(self.codes, self.cprime, self.levels)

    def dequant_f16(self) -> np.ndarray:
        """fp64 values of the fp16 dequantized weight (reading R11)."""
        return fp16_round(scaled_levels(self.codes, self.cprime, self.levels))


def packed_bytes(n: int, k: int, double_quant: bool = True, scale_bits: int = 32) -> int:
    """Bytes of one encoded weight: codes + code8 + s2 + mean, or codes + one
    fp32 (or bf16: scale_bits 16) scale per block without double
    quantization (codebook excluded)."""
    nb = n * k // BLOCK
    if not double_quant:
        return n * k // 2 + scale_bits // 8 * nb
    nc = -(-nb // DQ_BLOCK)
    return n * k // 2 + nb + 4 * nc + 4


def bits_per_weight(double_quant: bool = True, scale_bits: int = 32) -> float:
    """Storage per weight in the limit of many blocks: 4-bit code plus the
    amortized first-level constant, either kept at ``scale_bits`` or, with
    double quantization, as 8 bits per block plus one fp32 per 256 blocks."""
    if not double_quant:
        return 4.0 + scale_bits / BLOCK
    return 4.0 + 8.0 / BLOCK + 32.0 / (BLOCK * DQ_BLOCK)

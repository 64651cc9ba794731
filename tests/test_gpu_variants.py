"""GPU parity of the ablation variants: the uniform INT4 grid and the
encoding without double quantization, with fp32 or bf16 block scales
("QLoRA: Quantized Low-Rank Adaptation" (completesystemdesign.dev), "NF4: a
4-bit format matched to weight statistics", the worked block's scale "in
BF16" and the 65B arithmetic's one BF16 scalar per block; "QLoRA Explained
..." (gamut.so), "Double Quantization").

The kernels take the 16 levels from the weight's codebook and decode either
scale form, so each variant runs the same kernels as NF4 with double
quantization. For NF4 without double quantization (fp32 and bf16 block
scales) and for the uniform grid with and without it:
* the encoding is compared bit for bit with the oracle's (codes; code8, s2,
  mean, or the fp32 / bf16 block scales) and so is every dequantized bf16
  weight, also from fp32 weights whose absmax is no bf16 number;
* the layer (qlora_linear_fwd / _bwd) on the GEMV, fused and expanded paths
  against the fp64 oracle over the variant's own dequantized weight (relative
  Frobenius error <= 2e-3 and the element-wise bound for Y and dX, 1e-5 for
  the fp32 adapter gradients);
* the adapter merge within the merge's bracket bar.
"""

import numpy as np
import pytest
import torch

from bit_nf4_quantized_02_amd import synth
from oracle import linear as olin
from oracle import nf4 as onf4

from gpu_util import TOL, assert_dx, assert_fwd, assert_grad, bits16, f32, report, say
from test_gpu_merge import _bracket

pytestmark = pytest.mark.gpu

# (grid, double quantization, block-scale dtype without it)
VARIANTS = [("nf4", False, "fp32"), ("nf4", False, "bf16"), ("uniform", True, "fp32"), ("uniform", False, "fp32"),
            ("uniform", False, "bf16")]


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_02_amd import qlora
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return qlora


def _levels(grid):
    return onf4.nf4_levels() if grid == "nf4" else onf4.uniform4_levels()


def _encode(q, W, grid, dq, sd="fp32"):
    cb = q.build_nf4_codebook() if grid == "nf4" else q.build_uniform4_codebook()
    gw = q.quantize_nf4(W.cuda(), codebook=torch.tensor(cb, dtype=torch.float32, device="cuda"), double_quant=dq,
                        scale_dtype=torch.bfloat16 if sd == "bf16" else torch.float32)
    ow = onf4.NF4Weight(W.float().numpy(), _levels(grid), double_quant=dq, scale_dtype=sd)
    return gw, ow


@pytest.mark.parametrize("grid,dq,sd", VARIANTS)
@pytest.mark.parametrize("n,k,wdt", [(37, 192, "bf16"), (300, 4096, "bf16"), (257, 320, "bf16"), (129, 448, "fp32")])
def test_encode_and_dequant_bitwise(q, grid, dq, sd, n, k, wdt):
    say(f"case: encode {grid} double_quant={dq} scales={sd} n={n} k={k} W {wdt}")
    W = synth.weight_bf16(n, k, 0.02, 71, n, k).float()
    W[n // 2, 64:128] = 0.0                       # an all-zero block
    if wdt == "fp32":
        # fp32 weights: block maxima that are no bf16 number (rounding up and down)
        W[::3, 5] = 0.0501
        W[1::3, 70] = -0.0507
        W[:, 200] *= 1.0 + 2.0 ** -12
    else:
        W = W.to(torch.bfloat16)
    gw, ow = _encode(q, W, grid, dq, sd)
    wd = q.dequant(gw)
    torch.cuda.synchronize()
    assert np.array_equal(gw.codes.cpu().numpy(), ow.packed), "packed codes differ"
    if dq:
        assert np.array_equal(gw.code8.cpu().numpy(), ow.code8), "code8 differs"
        assert np.array_equal(gw.s2.cpu().numpy().view(np.uint32), ow.s2.view(np.uint32)), "s2 differs"
        assert gw.mean.cpu().numpy().view(np.uint32)[0] == np.float32(ow.mean).view(np.uint32)
    elif sd == "bf16":
        assert gw.code8 is None and gw.mean is None and gw.s2.dtype == torch.bfloat16
        assert np.array_equal(bits16(gw.s2), ow.s2), "bf16 block scales differ"
    else:
        assert gw.code8 is None and gw.mean is None
        assert np.array_equal(gw.s2.cpu().numpy().view(np.uint32), ow.s2.view(np.uint32)), "block scales differ"
    assert np.array_equal(bits16(wd), ow.dequant_bits()), "dequantized bf16 differs"
    assert gw.nbytes() == onf4.packed_bytes(n, k, double_quant=dq, scale_bits=16 if sd == "bf16" else 32)


@pytest.mark.parametrize("grid,dq,sd", VARIANTS)
@pytest.mark.parametrize("m", [4, 64, 512])
def test_layer_on_every_path(q, grid, dq, sd, m):
    n, k, r, s = 520, 640, 16, 2.0
    paths = (q.linear_path(m, n, k, r, False), q.linear_path(m, n, k, r, True))
    say(f"case: layer {grid} double_quant={dq} scales={sd} M={m} N={n} K={k} r={r} paths fwd/bwd={paths}")
    li = synth.linear_inputs(81, m, 0, n, k, m, r, s, sigma=0.02)
    gw, ow = _encode(q, li.W, grid, dq, sd)
    X, dY, A, B = li.X.cuda(), li.dY.cuda(), li.A.cuda(), li.B.cuda()
    Y, T = q.linear_fwd(gw, X, A, B, s)
    dX, dA, dB = q.linear_bwd(gw, X, T, dY, A, B, s)
    torch.cuda.synchronize()
    Wd = ow.dequant().astype(np.float64)
    Xo, Ao, Bo, dYo = (t.float().numpy().astype(np.float64) for t in (li.X, li.A, li.B, li.dY))
    Yr, _ = olin.linear_fwd(Xo, Wd, Ao, Bo, s)
    dXr, dAr, dBr, _ = olin.linear_bwd(Xo, Wd, Ao, Bo, s, dYo)
    assert_fwd("Y", Y, Xo, Wd, Ao, Bo, s, Yr)
    assert_dx("dX", dX, dYo, Wd, Ao, Bo, s, dXr)
    assert_grad("dA", dA, dAr)
    assert_grad("dB", dB, dBr)


@pytest.mark.parametrize("grid,dq,sd", VARIANTS)
def test_merge(q, grid, dq, sd):
    n, k, r, s = 200, 320, 8, 2.0
    say(f"case: merge {grid} double_quant={dq} scales={sd} n={n} k={k} r={r}")
    li = synth.linear_inputs(82, 0, 0, n, k, 1, r, s, sigma=0.02)
    gw, ow = _encode(q, li.W, grid, dq, sd)
    m16 = q.adapter_merge(gw, li.A.cuda(), li.B.cuda(), s)
    torch.cuda.synchronize()
    _bracket(f32(m16).astype(np.float64), ow.dequant().astype(np.float64), li.A.float().numpy(),
             li.B.float().numpy(), s, r, "bf16")


@pytest.mark.parametrize("grid,sd", [("uniform", "fp32"), ("nf4", "bf16")])
def test_decode_gemv_at_full_size_without_double_quant(q, grid, sd):
    """The 70B-class down weight (8192 x 28672, 8 waves per workgroup)
    without double quantization at M = 16: every output."""
    n, k, r, M = 8192, 28672, 16, 16
    say(f"case: decode GEMV {grid}, no double quant, {sd} scales, {n}x{k} M={M}")
    W = synth.weight_bf16(n, k, 0.015, 83, 0, 0)
    gw, ow = _encode(q, W, grid, False, sd)
    li = synth.linear_inputs(83, 0, 1, 1, k, M, r, 1.0)
    X, A = li.X.cuda(), li.A.cuda()
    B = synth.lora_B(n, r, 83, 0, synth.T_B).cuda()
    Y, T = q.linear_fwd(gw, X, A, B, 1.0)
    torch.cuda.synchronize()
    Xo, Wd = li.X.float().numpy().astype(np.float64), ow.dequant().astype(np.float64)
    Ao, Bo = li.A.float().numpy().astype(np.float64), B.float().cpu().numpy().astype(np.float64)
    Yr, _ = olin.linear_fwd(Xo, Wd, Ao, Bo, 1.0)
    assert_fwd("Y", Y, Xo, Wd, Ao, Bo, 1.0, Yr)

"""GPU parity of the layer over a bf16 base weight (qlora_lora_linear_fwd /
_bwd), the LoRA layer the pages compare QLoRA with ("QLoRA Explained ..."
(gamut.so), "QLoRA vs LoRA: Memory, Speed, and Quality Tradeoffs"; "QLoRA:
Quantized Low-Rank Adaptation" (completesystemdesign.dev), "Two prices to
know"), against the fp64 oracle with W itself as the base:
relative Frobenius error <= 2e-3 and the element-wise bound for Y and dX,
1e-5 for T, dA, dB; ragged shapes, n % 8 != 0, r = 0 and the largest rank,
few tokens, contractions split over workgroups, and the 4096^3 projection.
With W = the dequantized NF4 weight and the QLoRA layer on its expanded path,
Y and dX are equal bit for bit (the same GEMM over the same values in the
same order: only where the weight tiles come from differs -- the expansion
in workspace, or W itself, read contraction-major for dX); T, dA, dB are
always equal (the same low-rank kernels).
"""

import numpy as np
import pytest
import torch

from bit_nf4_quantized_02_amd import synth
from oracle import linear as olin

from gpu_util import assert_dx, assert_fwd, assert_grad, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_02_amd import qlora
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return qlora


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,n,k,r", [
    (300, 200, 192, 8),       # ragged M and N
    (512, 384, 1024, 16),
    (257, 100, 640, 5),       # n % 8 != 0: dX reads dY element-wise, odd rank
    (16, 1000, 2048, 16),     # few tokens
    (3, 64, 64, 1),
    (640, 256, 512, 64),
    (256, 128, 256, 128),     # largest rank
    (300, 130, 320, 0),       # no low-rank branch
    (300, 520, 2048, 16),     # few output tiles, long contraction: split over workgroups
])
def test_bf16_base_layer_against_oracle(q, m, n, k, r):
    s = 2.0 if r else 0.0
    say(f"case: bf16-base layer M={m} N={n} K={k} r={r}")
    li = synth.linear_inputs(86, m + n, 0, n, k, m, r, s, sigma=0.02)
    W, X, dY = li.W.cuda(), li.X.cuda(), li.dY.cuda()
    A = li.A.cuda() if r else None
    B = li.B.cuda() if r else None
    Y, T = q.lora_linear_fwd(W, X, A, B, s)
    dX, dA, dB = q.lora_linear_bwd(W, X, T, dY, A, B, s)
    torch.cuda.synchronize()
    Wo, Xo, Ao, Bo, dYo = (_f64(t) for t in (li.W, li.X, li.A, li.B, li.dY))
    Yr, Tr = olin.linear_fwd(Xo, Wo, Ao, Bo, s)
    dXr, dAr, dBr, _ = olin.linear_bwd(Xo, Wo, Ao, Bo, s, dYo)
    assert_fwd("Y", Y, Xo, Wo, Ao, Bo, s, Yr)
    assert_dx("dX", dX, dYo, Wo, Ao, Bo, s, dXr)
    if r:
        assert_grad("T", T, Tr)
        assert_grad("dA", dA, dAr)
        assert_grad("dB", dB, dBr)


def test_bf16_base_recompute_T_and_accumulate(q):
    m, n, k, r, s = 200, 160, 256, 8, 2.0
    li = synth.linear_inputs(87, 0, 0, n, k, m, r, s, sigma=0.02)
    W, X, dY, A, B = (t.cuda() for t in (li.W, li.X, li.dY, li.A, li.B))
    _, T = q.lora_linear_fwd(W, X, A, B, s)
    _, dA1, dB1 = q.lora_linear_bwd(W, X, T, dY, A, B, s, need_dX=False)
    _, dA2, dB2 = q.lora_linear_bwd(W, X, None, dY, A, B, s, need_dX=False)
    _, dA3, dB3 = q.lora_linear_bwd(W, X, T, dY, A, B, s, need_dX=False, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dA1, dA2) and torch.allclose(dB1, dB2, rtol=0, atol=1e-6)
    assert torch.equal(dA3, dA1) and torch.equal(dB3, dB1)  # accumulate onto zeros


@pytest.mark.parametrize("m,n,k", [(64, 520, 640), (512, 520, 640), (300, 2056, 576)])
def test_bf16_base_equals_qlora_over_the_dequantized_weight(q, m, n, k):
    """W = the dequantized NF4 weight: where the QLoRA layer takes its
    expanded path (M >= 128; 2056 x 576 with few output tiles splits dX along
    the contraction) Y and dX agree bit for bit."""
    r, s = 16, 2.0
    say(f"case: bf16 base vs QLoRA over W' M={m} paths fwd/bwd="
        f"{q.linear_path(m, n, k, r, False)}/{q.linear_path(m, n, k, r, True)}")
    li = synth.linear_inputs(88, m, 0, n, k, m, r, s, sigma=0.02)
    gw = q.quantize_nf4(li.W.cuda())
    Wd = q.dequant(gw)
    X, dY, A, B = (t.cuda() for t in (li.X, li.dY, li.A, li.B))
    Yq, Tq = q.linear_fwd(gw, X, A, B, s)
    dXq, dAq, dBq = q.linear_bwd(gw, X, Tq, dY, A, B, s)
    Yb, Tb = q.lora_linear_fwd(Wd, X, A, B, s)
    dXb, dAb, dBb = q.lora_linear_bwd(Wd, X, Tb, dY, A, B, s)
    torch.cuda.synchronize()
    assert torch.equal(Tq, Tb) and torch.equal(dAq, dAb) and torch.equal(dBq, dBb)
    if q.linear_path(m, n, k, r, False) == q.PATH_EXPANDED:
        assert torch.equal(Yq, Yb)
    if q.linear_path(m, n, k, r, True) == q.PATH_EXPANDED:
        assert torch.equal(dXq, dXb)


def test_bf16_base_at_the_attention_projection_size(q):
    """4096 x 4096, M = 4096, r = 16: every output."""
    c = synth.CONFIGS[2]
    li = synth.config_linear_inputs(2)
    say(f"case: bf16-base layer, {c.title}")
    W, X, dY, A, B = (t.cuda() for t in (li.W, li.X, li.dY, li.A, li.B))
    Y, T = q.lora_linear_fwd(W, X, A, B, li.scale)
    dX, dA, dB = q.lora_linear_bwd(W, X, T, dY, A, B, li.scale)
    torch.cuda.synchronize()
    Wo, Xo, Ao, Bo, dYo = (_f64(t) for t in (li.W, li.X, li.A, li.B, li.dY))
    Yr, _ = olin.linear_fwd(Xo, Wo, Ao, Bo, li.scale)
    dXr, dAr, dBr, _ = olin.linear_bwd(Xo, Wo, Ao, Bo, li.scale, dYo)
    assert_fwd("Y", Y, Xo, Wo, Ao, Bo, li.scale, Yr)
    assert_dx("dX", dX, dYo, Wo, Ao, Bo, li.scale, dXr)
    assert_grad("dA", dA, dAr)
    assert_grad("dB", dB, dBr)

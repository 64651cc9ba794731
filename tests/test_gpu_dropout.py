"""GPU parity of the layer with dropout on the adapter's input (LoRA dropout
0.05, "QLoRA Explained ..." (gamut.so), "Step 3: Configure and Apply LoRA
Adapters"): qlora_linear_fwd_dropout / _bwd_dropout against the fp64 oracle
(``linear_fwd_dropout`` / ``linear_bwd_dropout``) on the GEMV, fused and
expanded paths, with ragged shapes and a dX whose last-wave tiles are split
along the contraction; the saved T against (X . mask) A^T; and the special
masks (keep everything: the forward equals the plain layer bit for bit; drop
everything: the adapter gradients are exactly zero and dX is the base term).
Bars: relative Frobenius error <= 2e-3 for Y and dX with every element of
them inside the oracle's element-wise bound (low-rank term through the mask);
1e-5 for the fp32 T, dA and dB.
"""

import numpy as np
import pytest
import torch

from bit_nf4_quantized_02_amd import synth
from oracle import linear as olin

from gpu_util import TOL, assert_dx, assert_fwd, assert_grad, f32, oracle_encode, report, say

pytestmark = pytest.mark.gpu

P = 0.05
KEEP = 1.0 / (1.0 - P)


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_02_amd import qlora
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return qlora


def _run(q, m, n, k, r, s, mask_kind="drawn", seed=0):
    li = synth.linear_inputs(84, m + seed, 0, n, k, m, r, s, sigma=0.02)
    if mask_kind == "drawn":
        mask = synth.dropout_mask(m, k, P, 84, m, n, k, seed)
    elif mask_kind == "ones":
        mask = torch.ones((m, k), dtype=torch.uint8)
    else:
        mask = torch.zeros((m, k), dtype=torch.uint8)
    gw = q.quantize_nf4(li.W.cuda())
    X, dY, A, B, Md = li.X.cuda(), li.dY.cuda(), li.A.cuda(), li.B.cuda(), mask.cuda()
    Y, T = q.linear_fwd_dropout(gw, X, A, B, s, Md, KEEP)
    dX, dA, dB = q.linear_bwd_dropout(gw, X, T, dY, A, B, s, Md, KEEP)
    torch.cuda.synchronize()
    return li, mask, gw, (X, dY, A, B, Md), (Y, T, dX, dA, dB)


@pytest.mark.parametrize("m,n,k,r", [
    (4, 300, 512, 16),        # GEMV forward, fused dX
    (64, 520, 640, 16),       # fused forward and dX
    (512, 264, 640, 64),      # expanded forward and dX, ragged n
    (300, 2056, 576, 16),     # expanded, dX with last-wave tiles split along the contraction
    (130, 77, 192, 3),        # fused dX (n % 8 != 0), odd rank
])
def test_dropout_layer_against_oracle(q, m, n, k, r):
    s = 2.0
    say(f"case: dropout M={m} N={n} K={k} r={r} paths fwd/bwd="
        f"{q.linear_path(m, n, k, r, False)}/{q.linear_path(m, n, k, r, True)}")
    li, mask, _, _, (Y, T, dX, dA, dB) = _run(q, m, n, k, r, s)
    Wd = oracle_encode(li.W).dequant()
    Xo, Ao, Bo, dYo = (t.float().numpy().astype(np.float64) for t in (li.X, li.A, li.B, li.dY))
    mo = mask.numpy()
    Yr, Tdr = olin.linear_fwd_dropout(Xo, Wd, Ao, Bo, s, mo, KEEP)
    dXr, dAr, dBr, _ = olin.linear_bwd_dropout(Xo, Wd, Ao, Bo, s, dYo, mo, KEEP)
    assert_fwd("Y", Y, Xo, Wd, Ao, Bo, s, Yr, mask=mo, keep_scale=KEEP)
    assert_grad("T (X . mask) A^T", T, Tdr / KEEP)
    assert_dx("dX", dX, dYo, Wd, Ao, Bo, s, dXr, mask=mo, keep_scale=KEEP)
    assert_grad("dA", dA, dAr)
    assert_grad("dB", dB, dBr)


def test_keep_everything_matches_the_plain_forward(q):
    m, n, k, r, s = 512, 256, 512, 16, 2.0
    say("case: dropout mask all ones, keep scale 1")
    li = synth.linear_inputs(85, 0, 0, n, k, m, r, s, sigma=0.02)
    gw = q.quantize_nf4(li.W.cuda())
    X, A, B, dY = li.X.cuda(), li.A.cuda(), li.B.cuda(), li.dY.cuda()
    ones = torch.ones((m, k), dtype=torch.uint8, device="cuda")
    Y1, T1 = q.linear_fwd_dropout(gw, X, A, B, s, ones, 1.0)
    Y0, T0 = q.linear_fwd(gw, X, A, B, s)
    dX1, dA1, dB1 = q.linear_bwd_dropout(gw, X, T1, dY, A, B, s, ones, 1.0)
    dX0, dA0, dB0 = q.linear_bwd(gw, X, T0, dY, A, B, s)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y0) and torch.equal(T1, T0)
    assert torch.equal(dA1, dA0) and torch.equal(dB1, dB0)
    # dX adds the low-rank term first here: same sum, another order
    d = (dX1.float() - dX0.float()).abs().max().item()
    say(f"  dX max |diff| {d:.3e}")
    assert d <= 2.0 ** -6 * dX0.float().abs().max().item()


@pytest.mark.parametrize("m", [16, 512])
def test_drop_everything_leaves_the_base(q, m):
    n, k, r, s = 264, 512, 16, 2.0
    say(f"case: dropout mask all zeros M={m}")
    li, _, _, _, (Y, T, dX, dA, dB) = _run(q, m, n, k, r, s, mask_kind="zeros", seed=1)
    assert not T.any() and not dA.any() and not dB.any()
    Wd = oracle_encode(li.W).dequant()
    Xo, dYo = li.X.float().numpy().astype(np.float64), li.dY.float().numpy().astype(np.float64)
    assert report("Y (base only)", f32(Y), Xo @ Wd.T) <= TOL
    assert report("dX (base only)", f32(dX), dYo @ Wd) <= TOL


def test_dropout_at_the_attention_projection_size(q):
    """4096 x 4096, M = 4096, r = 16 (the default bench workload): every output."""
    m = n = k = 4096
    r, s = 16, 2.0
    say("case: dropout 4096^3 r=16")
    li, mask, _, _, (Y, T, dX, dA, dB) = _run(q, m, n, k, r, s, seed=2)
    Wd = oracle_encode(li.W).dequant()
    Xo, Ao, Bo, dYo = (t.float().numpy().astype(np.float64) for t in (li.X, li.A, li.B, li.dY))
    mo = mask.numpy()
    Yr, _ = olin.linear_fwd_dropout(Xo, Wd, Ao, Bo, s, mo, KEEP)
    dXr, dAr, dBr, _ = olin.linear_bwd_dropout(Xo, Wd, Ao, Bo, s, dYo, mo, KEEP)
    assert_fwd("Y", Y, Xo, Wd, Ao, Bo, s, Yr, mask=mo, keep_scale=KEEP)
    assert_dx("dX", dX, dYo, Wd, Ao, Bo, s, dXr, mask=mo, keep_scale=KEEP)
    assert_grad("dA", dA, dAr)
    assert_grad("dB", dB, dBr)

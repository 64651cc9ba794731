"""GPU parity of the low-rank kernels alone, against the fp64 oracle.

qlora_lowrank_project (T = X A^T with A as [r, C]; U = dY B with B as
[C, r]) and qlora_lowrank_grad (dA = s U^T X as [r, C]; dB = s dY^T T as
[C, r]) on the same bf16 / fp32 inputs the oracle evaluates in fp64. Bar:
relative Frobenius error <= 1e-5 (bf16 products, fp32 sums; the gradients
take their fp32 Q as a bf16 hi/lo pair). The projection's split output is
checked bit for bit against RN_bf16 of the kernel's own scaled fp32 result
(hi) and of the remainder (lo), zero past 2r.

Shapes reach every launch form: 64-row workgroups with contraction splits
(from 2048 rows, ranks 17..64), 16-row workgroups (smaller M or r <= 16),
ragged row and column tails, rows whose length is not a multiple of 8
(element-wise loads), and the token-split gradient path; in the 64-row form
also waves with 1, 2, 4 and 5 column batches and waves with none.
"""

import numpy as np
import pytest
import torch

from oracle import linear as olin

from gpu_util import GTOL, f32, report, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_02_amd import qlora
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return qlora


def _bf16(shape, scale, gen):
    return (torch.randn(shape, generator=gen) * scale).to(torch.bfloat16)


SHAPES = [
    (2048, 4096, 64),    # 64-row workgroups, whole tiles
    (2085, 4168, 33),    # ragged rows (37 past a multiple of 64) and columns (C % 32 = 8)
    (2085, 4170, 64),    # C % 8 != 0: element-wise loads on the tall path
    (4096, 8192, 64),    # the 65B-class stack's shape
    (2048, 4096, 16),    # r <= 16: 16-row workgroups at large M
    (300, 1000, 24),     # small M: 16-row workgroups, contraction split over workgroups
    (16, 1024, 8),       # decode-sized
    (2048, 304, 40),     # 64-row form, short contraction: waves with one and two column batches
    (2112, 40, 64),      # 64-row form, 40 columns: most waves get no batch at all
]


@pytest.mark.parametrize("m,c,r", SHAPES)
def test_project_against_oracle(q, m, c, r):
    say(f"case: project M={m} C={c} r={r}")
    g = torch.Generator().manual_seed(m * 7 + c * 3 + r)
    P = _bf16((m, c), 1.0, g)
    A = _bf16((r, c), c ** -0.5, g)
    B = _bf16((c, r), 0.01, g)
    s = 0.25
    Pd, Ad, Bd = P.cuda(), A.cuda(), B.cuda()
    T, TS = q.lowrank_project(Pd, Ad, 0, s, want_out=True, want_split=True)
    U, US = q.lowrank_project(Pd, Bd, 1, s, want_out=True, want_split=True)
    torch.cuda.synchronize()
    Po, Ao, Bo = (t.float().numpy() for t in (P, A, B))
    # the oracle's T = X A^T (its linear_fwd with a one-row zero base) and
    # U = dY B (its adapter gradients with a one-column zero X)
    _, Tr = olin.linear_fwd(Po, np.zeros((1, c)), Ao, np.zeros((1, r)), s)
    _, _, Ur = olin.adapter_grads(np.zeros((m, 1)), np.zeros((r, 1)), Bo, s, Po, T=np.zeros((m, r)))
    assert report("T", f32(T), Tr, floor=False) <= GTOL
    assert report("U", f32(U), Ur, floor=False) <= GTOL
    xc = q.lowrank_split_cols(r)
    for name, out, split in (("T", T, TS), ("U", U, US)):
        sv = out.cpu() * s
        hi = sv.to(torch.bfloat16)
        lo = (sv - hi.float()).to(torch.bfloat16)
        sp = split.cpu()
        assert sp.shape == (m, xc)
        assert torch.equal(sp[:, :r].view(torch.int16), hi.view(torch.int16)), f"{name} split hi"
        assert torch.equal(sp[:, r:2 * r].view(torch.int16), lo.view(torch.int16)), f"{name} split lo"
        assert not sp[:, 2 * r:].float().abs().sum().item(), f"{name} split pad"


@pytest.mark.parametrize("m,c,r", SHAPES)
def test_grad_against_oracle(q, m, c, r):
    say(f"case: grad M={m} C={c} r={r}")
    g = torch.Generator().manual_seed(m * 5 + c * 11 + r)
    P = _bf16((m, c), 1.0, g)
    Qv = torch.randn((m, r), generator=g)
    s = 0.25
    Pd, Qd = P.cuda(), Qv.cuda()
    dA = q.lowrank_grad(Pd, Qd, s, 0)
    dB = q.lowrank_grad(Pd, Qd, s, 1)
    torch.cuda.synchronize()
    Po, Qo = P.float().numpy(), Qv.numpy()
    # dA = s U^T X with U = Q (the oracle's adapter gradients with B = I)
    dAr, _, _ = olin.adapter_grads(Po, np.zeros((r, c)), np.eye(r), s, Qo, T=np.zeros((m, r)))
    # dB = s dY^T T with dY = P, T = Q
    _, dBr, _ = olin.adapter_grads(np.zeros((m, 1)), np.zeros((r, 1)), np.zeros((c, r)), s, Po, T=Qo)
    assert report("dA", f32(dA), dAr, floor=False) <= GTOL
    assert report("dB", f32(dB), dBr, floor=False) <= GTOL


def test_project_reruns_are_bit_identical(q):
    g = torch.Generator().manual_seed(5)
    P = _bf16((2085, 4168), 1.0, g).cuda()
    A = _bf16((64, 4168), 0.02, g).cuda()
    T1, S1 = q.lowrank_project(P, A, 0, 0.5, want_split=True)
    T2, S2 = q.lowrank_project(P, A, 0, 0.5, want_split=True)
    torch.cuda.synchronize()
    assert torch.equal(T1, T2) and torch.equal(S1, S2)

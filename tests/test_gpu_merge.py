"""GPU parity of the adapter merge and unmerge (qlora_adapter_merge /
qlora_adapter_unmerge) against the fp64 oracle.

Bar, derived from the arithmetic (one fp32 sum of r exact products on the
matrix cores, one fp32 multiply by s, one fp32 addition, then one rounding):
every fp32 value v the kernel can form satisfies
    |v - exact| <= eps = (r + 3) * 2^-24 * (|W'| + |s| * sum_j |B A|),
so a bf16 output must lie between round_bf16(exact - eps) and
round_bf16(exact + eps) (it equals round_bf16(exact) unless the exact value
is within eps of a rounding midpoint), and an fp32 output within eps of the
exact value. Shapes cover partial tiles (n % 64, k % 128), ranks 1 .. 128
(including r % 8 != 0 and the no-adapter case) and the 4096x4096 and
11008x4096 weights at full size.
"""

import numpy as np
import pytest
import torch

from oracle import merge as omerge

from gpu_util import f32, oracle_encode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_02_amd import qlora
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return qlora


def _inputs(n, k, r, seed):
    g = torch.Generator().manual_seed(seed)
    W = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    A = (torch.rand(r, k, generator=g) * 2 - 1).div(k ** 0.5).to(torch.bfloat16) if r else None
    B = (torch.randn(n, r, generator=g) * 0.01).to(torch.bfloat16) if r else None
    return W, A, B


def _bracket(got, Wd, A, B, s, r, kind, sign=1.0):
    """Check got (fp64 values) against exact = Wd + sign*s*B A within the bar."""
    Wd = np.asarray(Wd, dtype=np.float64)
    if r:
        A64, B64 = A.astype(np.float64), B.astype(np.float64)
        exact = Wd + sign * s * (B64 @ A64)
        mag = np.abs(Wd) + abs(s) * (np.abs(B64) @ np.abs(A64))
    else:
        exact, mag = Wd, np.abs(Wd)
    eps = (r + 3) * 2.0 ** -24 * mag
    if kind == "fp32":
        bad = np.abs(got - exact) > eps
    else:
        lo, hi = omerge.round_bf16(exact - eps), omerge.round_bf16(exact + eps)
        bad = (got < lo) | (got > hi)
        same = np.mean(got == omerge.round_bf16(exact))
        say(f"    equal to round_bf16(exact): {same * 100:.4f}%")
        assert same > 0.99
    say(f"    outside the bar: {int(bad.sum())} of {bad.size}")
    assert not bad.any()


@pytest.mark.parametrize("n,k,r", [(128, 256, 16), (200, 320, 8), (64, 64, 1), (300, 1024, 64), (96, 192, 128),
                                   (130, 448, 12), (64, 128, 0)])
def test_merge_and_unmerge_small(q, n, k, r):
    s = 2.0 if r else 0.0
    say(f"case: merge n={n} k={k} r={r} s={s}")
    W, A, B = _inputs(n, k, r, n * 1000 + k + r)
    gw = q.quantize_nf4(W.cuda())
    Ad = A.cuda() if r else None
    Bd = B.cuda() if r else None
    m16 = q.adapter_merge(gw, Ad, Bd, s)
    m32 = q.adapter_merge(gw, Ad, Bd, s, out_dtype=torch.float32)
    deq = q.dequant(gw)
    back = q.adapter_unmerge(m16, Ad, Bd, s)
    torch.cuda.synchronize()
    Wd = oracle_encode(W).dequant().astype(np.float64)
    assert np.array_equal(f32(deq).astype(np.float64), Wd)   # the base the merge adds onto
    An = A.float().numpy() if r else None
    Bn = B.float().numpy() if r else None
    say("  bf16 merge")
    _bracket(f32(m16).astype(np.float64), Wd, An, Bn, s, r, "bf16")
    say("  fp32 merge")
    _bracket(f32(m32).astype(np.float64), Wd, An, Bn, s, r, "fp32")
    say("  unmerge of the GPU's bf16 merge")
    _bracket(f32(back).astype(np.float64), f32(m16).astype(np.float64), An, Bn, s, r, "bf16", sign=-1.0)
    if r == 0:
        assert torch.equal(m16, deq)
    # in place
    q.adapter_unmerge(m16, Ad, Bd, s, out=m16)
    torch.cuda.synchronize()
    assert torch.equal(m16, back)


@pytest.mark.parametrize("n,k,r", [(4096, 4096, 16), (11008, 4096, 64)])
def test_merge_full_size(q, n, k, r):
    s = 2.0 if r == 16 else 0.25
    say(f"case: merge full size n={n} k={k} r={r}")
    W, A, B = _inputs(n, k, r, 99 + r)
    gw = q.quantize_nf4(W.cuda())
    m16 = q.adapter_merge(gw, A.cuda(), B.cuda(), s)
    torch.cuda.synchronize()
    Wd = oracle_encode(W).dequant().astype(np.float64)
    _bracket(f32(m16).astype(np.float64), Wd, A.float().numpy(), B.float().numpy(), s, r, "bf16")

"""Shared helpers of the GPU parity tests (imported by tests only)."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import linear as olin
from oracle import nf4 as onf4

TOL = 2e-3          # relative Frobenius error bar for bf16 outputs and fp32 gradients


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").float().numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_encode(W_host: torch.Tensor) -> onf4.NF4Weight:
    """The oracle's own encoding of the bf16 (or fp32) input weight."""
    return onf4.NF4Weight(W_host.float().numpy())


def assert_encode_equal(gw, ow: onf4.NF4Weight, rows=None):
    codes = gw.codes.cpu().numpy()
    if rows is None:
        assert np.array_equal(codes, ow.packed), "packed codes differ"
        assert np.array_equal(gw.code8.cpu().numpy(), ow.code8), "code8 differs"
    else:
        assert np.array_equal(codes[rows], ow.packed[rows]), "packed codes differ"
    assert np.array_equal(gw.s2.cpu().numpy().view(np.uint32), ow.s2.view(np.uint32)), "s2 differs"
    assert gw.mean.cpu().numpy().view(np.uint32)[0] == np.float32(ow.mean).view(np.uint32), "mean differs"


def report(name, got, ref, floor=True):
    e = olin.relerr(got, ref)
    fl = olin.bf16_floor(ref) if floor else 0.0
    say(f"  {name}: relerr {e:.3e} (bf16 floor {fl:.3e})")
    return e


GTOL = 1e-5         # fp32 T and adapter gradients: the bf16 hi/lo split keeps them near 2.5e-6


def check_elementwise(name, got, ref, bound):
    """Every element of got within ref +- bound (the oracle's element-wise
    error bound of an fp32-accumulated 16-bit result); prints the worst
    ratio and returns the number of elements outside."""
    g = np.asarray(got, dtype=np.float64)
    d = np.abs(g - np.asarray(ref, dtype=np.float64))
    ratio = float(np.max(d / bound)) if d.size else 0.0
    bad = olin.outside_bound(g, ref, bound)
    say(f"  {name}: element-wise worst |err| / bound {ratio:.3f}, {bad} outside")
    return bad


def assert_fwd(name, Y, Xo, Wd, Ao, Bo, s, Yr, **kw):
    """Y against the oracle's Yr: relative Frobenius error <= TOL and every
    element inside the element-wise bound."""
    y = f32(Y)
    assert report(name, y, Yr) <= TOL
    assert check_elementwise(name, y, Yr, olin.fwd_error_bound(Xo, Wd, Ao, Bo, s, Yr, **kw)) == 0


def assert_dx(name, dX, dYo, Wd, Ao, Bo, s, dXr, **kw):
    """dX against the oracle's dXr, as assert_fwd."""
    d = f32(dX)
    assert report(name, d, dXr) <= TOL
    assert check_elementwise(name, d, dXr, olin.dx_error_bound(dYo, Wd, Ao, Bo, s, dXr, **kw)) == 0


def assert_grad(name, got, ref):
    """fp32 adapter gradient (or T) against the oracle: relative Frobenius
    error <= GTOL."""
    assert report(name, f32(got), ref, floor=False) <= GTOL

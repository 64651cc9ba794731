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

"""The forward that allocates nothing (qlora_linear_fwd_scratch), called
through the C ABI: its outputs equal qlora_linear_fwd's on the same inputs
bit for bit (same kernels, the library's own scratch as workspace) and are
within the parity bar of the oracle, on calls in a row that change the
kernel path and shrink the problem, so the second call meets the contents
the first left in the shared scratch. A request beyond the scratch size is
refused before anything is launched.
"""

import ctypes

import numpy as np
import pytest
import torch

from bit_nf4_quantized_02_amd import synth
from oracle import linear as olin

from gpu_util import assert_fwd, assert_grad, oracle_encode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_02_amd import qlora
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return qlora


def _call_both(q, li):
    m, n, k, r, s = li.meta["m"], li.meta["n"], li.meta["k"], li.meta["r"], li.scale
    say(f"case: scratch forward M={m} N={n} K={k} r={r} path={q.linear_path(m, n, k, r, False)}")
    gw = q.quantize_nf4(li.W.cuda())
    X, A, B = li.X.cuda(), li.A.cuda(), li.B.cuda()
    Y0, T0 = q.linear_fwd(gw, X, A, B, s)
    # the C ABI directly, outputs preallocated: nothing is allocated by the call
    Y1 = torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda")
    T1 = torch.full((m, r), 7.0, dtype=torch.float32, device="cuda")
    st = gw.struct()
    lib = q.raw()
    status = lib.qlora_linear_fwd_scratch(ctypes.byref(st), q._ptr(X), m, q._ptr(A), q._ptr(B), r, float(s),
                                          q._ptr(Y1), q._ptr(T1), q._stream())
    assert status == 0, q.status_string(status)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y0) and torch.equal(T1, T0)
    Wd = oracle_encode(li.W).dequant()
    Xo, Ao, Bo = (t.float().numpy().astype(np.float64) for t in (li.X, li.A, li.B))
    Yr, Tr = olin.linear_fwd(Xo, Wd, Ao, Bo, s)
    assert_fwd("Y", Y1, Xo, Wd, Ao, Bo, s, Yr)
    assert_grad("T", T1, Tr)


def test_scratch_forward_matches_the_workspace_forward(q):
    # expanded path (a 2.1 MB expansion in the scratch), then the fused path,
    # then the GEMV path on a smaller input: each call after one that left
    # larger contents behind
    _call_both(q, synth.linear_inputs(97, 0, 0, 1024, 1024, 512, 16, 2.0))
    _call_both(q, synth.linear_inputs(97, 1, 0, 520, 640, 64, 8, 2.0))
    _call_both(q, synth.linear_inputs(97, 2, 0, 300, 512, 4, 16, 2.0))


def test_scratch_forward_refuses_a_request_beyond_the_scratch(q):
    n = k = 8192
    M, r = 4096, 64
    need = q.linear_workspace_bytes(M, n, k, r, False)
    assert need > q.SCRATCH_BYTES
    w = q.NF4Weight.empty(64, 64)
    st = w.struct()
    st.n, st.k = n, k
    p = ctypes.c_void_p(1 << 24)
    status = q.raw().qlora_linear_fwd_scratch(ctypes.byref(st), p, M, p, p, r, 1.0, p, None, q._stream())
    assert q.status_string(status).startswith("QLORA_ERR_SCRATCH")

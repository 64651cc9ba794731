"""Host-only checks of the C ABI (no GPU needed, no kernel launched).

* the library loads and exports every function include/qlora.h declares;
* the host codebook equals the oracle's table bit for bit (the two are
  computed by different inverse-CDF methods and share no code);
* size queries agree with the oracle's storage arithmetic;
* argument errors come back as status codes before anything is enqueued;
* the oracle and the library stay independent (no imports either way).
"""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

from oracle import nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")


@pytest.fixture(scope="module")
def q():
    from bit_nf4_quantized_02_amd import qlora
    return qlora


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(q):
    names = _declared_functions()
    assert len(names) >= 10
    lib = q.raw()
    for nme in names:
        assert hasattr(lib, nme), nme


def test_host_codebook_matches_oracle_bitwise(q):
    lv = np.array(q.build_nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lv.view(np.uint32), nf4.nf4_levels().view(np.uint32))
    assert q.raw().qlora_build_nf4_codebook(None) == -1


def test_uniform_codebook_matches_oracle_bitwise(q):
    lv = np.array(q.build_uniform4_codebook(), dtype=np.float32)
    assert np.array_equal(lv.view(np.uint32), nf4.uniform4_levels().view(np.uint32))
    assert q.raw().qlora_build_uniform4_codebook(None) == -1


@pytest.mark.parametrize("n,k", [(1024, 1024), (4096, 4096), (11008, 4096), (4096, 11008), (8192, 28672),
                                 (3, 64), (5, 192), (22016, 8192)])
def test_packed_bytes_agree_with_oracle(q, n, k):
    assert q.nf4_packed_bytes(n, k) == nf4.packed_bytes(n, k)
    assert q.nf4_packed_bytes(n, k, double_quant=False) == nf4.packed_bytes(n, k, double_quant=False)
    assert q.quantize_workspace_bytes(n, k) > 0


def test_weight_without_double_quant_needs_no_code8_or_mean(q):
    """code8 = NULL selects the form without double quantization (mean is not
    read, may be NULL); with code8 set, mean is required. Checked on the host
    with M = 0, which returns before any launch."""
    lib = q.raw()
    p = ctypes.c_void_p(1 << 24)
    base = 1 << 20
    nodq = q._Weight(64, 128, base, None, base + 8192, None, base + 16384)
    assert lib.qlora_linear_fwd(ctypes.byref(nodq), p, 0, p, p, 8, 1.0, p, None, None, 0, None) == 0
    half = q._Weight(64, 128, base, base + 4096, base + 8192, None, base + 16384)
    assert lib.qlora_linear_fwd(ctypes.byref(half), p, 0, p, p, 8, 1.0, p, None, None, 0, None) == -1
    nos2 = q._Weight(64, 128, base, None, None, None, base + 16384)
    assert lib.qlora_linear_fwd(ctypes.byref(nos2), p, 0, p, p, 8, 1.0, p, None, None, 0, None) == -1
    assert lib.qlora_nf4_storage_bytes(64, 128, 3) == 0
    assert lib.qlora_nf4_storage_bytes(64, 128, q.SCALE_BF16) == 64 * 128 // 2 + 2 * 128
    assert q.nf4_packed_bytes(64, 128, double_quant=False, scale_dtype=torch.bfloat16) == \
        nf4.packed_bytes(64, 128, double_quant=False, scale_bits=16)
    # bf16 block scales: only without double quantization, flag 0 or 1
    bfs = q._Weight(64, 128, base, None, base + 8192, None, base + 16384, 1)
    assert lib.qlora_linear_fwd(ctypes.byref(bfs), p, 0, p, p, 8, 1.0, p, None, None, 0, None) == 0
    both = q._Weight(64, 128, base, base + 4096, base + 8192, base + 12288, base + 16384, 1)
    assert lib.qlora_linear_fwd(ctypes.byref(both), p, 0, p, p, 8, 1.0, p, None, None, 0, None) == -1
    bad = q._Weight(64, 128, base, None, base + 8192, None, base + 16384, 2)
    assert lib.qlora_linear_fwd(ctypes.byref(bad), p, 0, p, p, 8, 1.0, p, None, None, 0, None) == -1


def test_size_queries_reject_bad_shapes(q):
    assert q.nf4_packed_bytes(4, 100) == 0
    assert q.nf4_packed_bytes(0, 64) == 0
    assert q.quantize_workspace_bytes(4, 65) == 0
    assert q.linear_workspace_bytes(16, 64, 100, 8, False) == 0
    assert q.linear_workspace_bytes(16, 64, 64, q.MAX_RANK + 1, True) == 0
    assert q.linear_workspace_bytes(0, 64, 64, 8, True) == 0
    assert q.linear_workspace_bytes(4096, 4096, 4096, 16, False) > 0
    assert q.linear_workspace_bytes(4096, 4096, 4096, 16, True) > 0
    # M <= 16 without a rank: only the activations in the GEMV operand order
    assert q.linear_workspace_bytes(16, 4096, 4096, 0, False) == q.nf4_gemv_workspace_bytes(4096)


def _fake_weight(q, n=64, k=128, aligned=True):
    base = 1 << 20
    off = 0 if aligned else 4
    return q._Weight(n, k, base + off, base + 4096, base + 8192, base + 12288, base + 16384)


def test_error_paths_return_before_any_launch(q):
    lib = q.raw()
    W = _fake_weight(q)
    p = ctypes.c_void_p(1 << 24)
    none = None
    # NULL weight
    assert lib.qlora_dequant(None, p, none) == -1
    assert lib.qlora_linear_fwd(None, p, 16, p, p, 8, 1.0, p, none, p, 1 << 20, none) == -1
    # K not a multiple of 64
    bad = _fake_weight(q, k=100)
    assert lib.qlora_dequant(ctypes.byref(bad), p, none) == -2
    assert lib.qlora_quantize_nf4(p, 0, ctypes.byref(bad), p, 1 << 20, none) == -2
    # misaligned buffer
    mis = _fake_weight(q, aligned=False)
    assert lib.qlora_dequant(ctypes.byref(mis), p, none) == -1
    assert lib.qlora_dequant(ctypes.byref(W), ctypes.c_void_p((1 << 24) + 2), none) == -1
    # bad dtype, too-small workspace
    assert lib.qlora_quantize_nf4(p, 7, ctypes.byref(W), p, 1 << 20, none) == -1
    assert lib.qlora_quantize_nf4(p, 0, ctypes.byref(W), p, 16, none) == -4
    need = q.linear_workspace_bytes(64, 64, 128, 8, False)
    assert lib.qlora_linear_fwd(ctypes.byref(W), p, 64, p, p, 8, 1.0, p, none, p, need - 1, none) == -4
    needb = q.linear_workspace_bytes(64, 64, 128, 8, True)
    assert lib.qlora_linear_bwd(ctypes.byref(W), p, none, p, 64, p, p, 8, 1.0, p, p, p, 0, p, needb - 1, none) == -4
    # rank out of range, negative M, bad accumulate flag, missing A/B
    assert lib.qlora_linear_fwd(ctypes.byref(W), p, 16, p, p, q.MAX_RANK + 1, 1.0, p, none, p, 1 << 30, none) == -2
    assert lib.qlora_linear_fwd(ctypes.byref(W), p, -1, p, p, 8, 1.0, p, none, p, 1 << 30, none) == -2
    assert lib.qlora_linear_bwd(ctypes.byref(W), p, none, p, 16, p, p, 8, 1.0, p, p, p, 2, p, 1 << 30, none) == -1
    assert lib.qlora_linear_fwd(ctypes.byref(W), p, 16, none, p, 8, 1.0, p, none, p, 1 << 30, none) == -1
    # M = 0 launches nothing and succeeds, except that a backward with
    # accumulate = 0 zeroes dA and dB (checked, then launched: GPU tests)
    assert lib.qlora_linear_fwd(ctypes.byref(W), p, 0, p, p, 8, 1.0, p, none, none, 0, none) == 0
    assert lib.qlora_linear_bwd(ctypes.byref(W), p, none, p, 0, p, p, 8, 1.0, p, p, p, 1, none, 0, none) == 0
    assert lib.qlora_linear_bwd(ctypes.byref(W), p, none, p, 0, p, p, 0, 1.0, p, p, p, 0, none, 0, none) == 0
    assert lib.qlora_linear_bwd(ctypes.byref(W), p, none, p, 0, p, p, 8, 1.0, p, ctypes.c_void_p((1 << 24) + 4),
                                p, 0, none, 0, none) == -1
    assert lib.qlora_silu_mul_fwd(p, p, p, 0, none) == 0
    assert lib.qlora_silu_mul_fwd(None, p, p, 8, none) == -1
    assert lib.qlora_silu_mul_bwd(p, p, p, p, p, -1, none) == -2
    for s in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(q.status_string(s), str) and q.status_string(s)


def test_oracle_and_library_are_independent():
    def imports(path):
        out = []
        for dp, _, files in os.walk(path):
            for f in files:
                if f.endswith((".py", ".hip", ".cpp", ".h")):
                    out.append((os.path.join(dp, f), open(os.path.join(dp, f)).read()))
        return out
    for path, text in imports(os.path.join(ROOT, "oracle")):
        assert "bit_nf4_quantized_02_amd" not in text, path
    for path, text in imports(os.path.join(ROOT, "bit_nf4_quantized_02_amd")):
        assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), path


def test_path_choice_and_expanded_sizes(q):
    # forward: GEMV up to 16 tokens, fused below the expansion threshold, expanded above
    assert q.linear_path(1, 4096, 4096, 16, False) == q.PATH_GEMV
    assert q.linear_path(16, 4096, 4096, 16, False) == q.PATH_GEMV
    assert q.linear_path(17, 4096, 4096, 16, False) == q.PATH_FUSED
    assert q.linear_path(127, 4096, 4096, 16, False) == q.PATH_FUSED
    assert q.linear_path(128, 4096, 4096, 16, False) == q.PATH_EXPANDED
    assert q.linear_path(16, 4096, 4096, 16, True) == q.PATH_GEMV   # dX through the GEMV for M <= 16
    assert q.linear_path(17, 4096, 4096, 16, True) == q.PATH_FUSED
    big = 4096
    assert q.linear_path(big, 4096, 4096, 16, False) == q.PATH_EXPANDED
    assert q.linear_path(big, 4096, 4096, 16, True) == q.PATH_EXPANDED
    # dX over unaligned dY rows (n % 8 != 0) stays on the fused kernel
    assert q.linear_path(big, 100, 4096, 16, True) == q.PATH_FUSED
    # the GEMV's 32-bit code offsets: a forward whose codes reach 4 GiB runs fused
    assert q.linear_path(16, 8192, 8192, 16, False) == q.PATH_GEMV
    assert q.linear_path(16, 1 << 20, 8192, 16, False) == q.PATH_FUSED
    assert q.linear_path(16, 1 << 20, 8192, 16, True) == q.PATH_GEMV
    assert q.linear_path(big, 100, 4096, 16, False) == q.PATH_EXPANDED
    with pytest.raises(q.QLoraError):
        q.linear_path(big, 64, 100, 16, False)
    # expanded operand sizes: [n, k + xc] and [k, roundup(n, 64) + xc] bf16 (256-B rounded)
    def r256(b):
        return (b + 255) // 256 * 256
    assert q.nf4_expand_bytes(4096, 4096, 16, False) == r256(4096 * (4096 + 64) * 2)
    assert q.nf4_expand_bytes(100, 256, 16, True) == r256(256 * (128 + 64) * 2)
    assert q.nf4_expand_bytes(100, 256, 0, True) == r256(256 * 128 * 2)
    assert q.nf4_expand_bytes(100, 255, 0, True) == 0
    # contraction-major dX operand: [n + xc, k], n % 64 == 0 only
    assert q.nf4_expand_bytes(4096, 4096, 16, 2) == r256((4096 + 64) * 4096 * 2)
    assert q.nf4_expand_bytes(4096, 4096, 0, 2) == r256(4096 * 4096 * 2)
    assert q.nf4_expand_bytes(100, 256, 16, 2) == 0
    assert q.nf4_expand_bytes(64, 256, 16, 3) == 0
    # the layer workspace grows by the expanded operand exactly when that path is taken
    fw_small = q.linear_workspace_bytes(64, 4096, 4096, 16, False)
    fw_big = q.linear_workspace_bytes(big, 4096, 4096, 16, False)
    assert fw_big - fw_small >= q.nf4_expand_bytes(4096, 4096, 16, False)


def test_expand_and_bf16_gemm_errors(q):
    lib = q.raw()
    W = _fake_weight(q)
    p = ctypes.c_void_p(1 << 24)
    need = q.nf4_expand_bytes(64, 128, 8, False)
    assert lib.qlora_nf4_expand(ctypes.byref(W), p, 8, 0, p, need - 1, None) == -4
    assert lib.qlora_nf4_expand(ctypes.byref(W), p, 8, 3, p, need, None) == -1
    need2 = q.nf4_expand_bytes(64, 128, 8, 2)
    assert lib.qlora_nf4_expand(ctypes.byref(W), p, 8, 2, p, need2 - 1, None) == -4
    assert lib.qlora_nf4_expand(ctypes.byref(W), None, 8, 0, p, need, None) == -1
    assert lib.qlora_nf4_expand(ctypes.byref(W), p, q.MAX_RANK + 1, 0, p, 1 << 30, None) == -2
    assert lib.qlora_bf16_gemm(p, 64, 100, p, 8, p, 64, p, None, 0, None) == -2      # kc % 8 != 0
    assert lib.qlora_bf16_gemm(p, 64, 128, None, 8, p, 64, p, None, 0, None) == -1   # r > 0 needs split
    assert lib.qlora_bf16_gemm(p, 0, 128, None, 8, p, 64, p, None, 0, None) == 0     # M = 0: no-op
    # few output tiles: split contraction, partial sums need workspace
    need = q.bf16_gemm_workspace_bytes(256, 4096, 8, 256)
    assert need >= 2 * 256 * 256 * 4
    assert lib.qlora_bf16_gemm(p, 256, 4096, p, 8, p, 256, p, None, 0, None) == -4
    assert lib.qlora_bf16_gemm(p, 256, 4096, p, 8, p, 256, p, p, need - 1, None) == -4
    assert q.bf16_gemm_workspace_bytes(4096, 4096, 16, 4096) == 0   # 256 tiles: whole contraction per tile
    # the contraction-major form: kc % 64 == 0 and nout % 8 == 0
    assert lib.qlora_bf16_gemm_nn(p, 64, 96, p, 8, p, 64, p, None, 0, None) == -2     # kc % 64 != 0
    assert lib.qlora_bf16_gemm_nn(p, 64, 128, p, 8, p, 100, p, None, 0, None) == -2   # nout % 8 != 0
    assert lib.qlora_bf16_gemm_nn(p, 64, 128, None, 8, p, 64, p, None, 0, None) == -1  # r > 0 needs split
    assert lib.qlora_bf16_gemm_nn(p, 0, 128, None, 8, p, 64, p, None, 0, None) == 0    # M = 0: no-op
    assert lib.qlora_bf16_gemm_nn(p, 256, 4096, p, 8, p, 256, p, None, 0, None) == -4  # split needs workspace


def test_expanded_path_needs_operands_under_4gib(q):
    lib = q.raw()
    p = ctypes.c_void_p(1 << 24)
    huge_m = 1 << 20  # [2^20, 4096] bf16 activation = 8 GiB
    assert q.linear_path(huge_m, 4096, 4096, 16, False) == q.PATH_FUSED
    assert q.linear_path(huge_m, 4096, 4096, 16, True) == q.PATH_FUSED
    assert lib.qlora_bf16_gemm(p, huge_m, 4096, p, 16, p, 4096, p, None, 0, None) == -2


def test_calibration_probe_errors(q):
    lib = q.raw()
    p = ctypes.c_void_p(1 << 24)
    assert lib.qlora_calib_mfma(0, 10, p, None) == -1
    assert lib.qlora_calib_mfma(4, 0, p, None) == -1
    assert lib.qlora_calib_mfma(4, 10, None, None) == -1
    assert lib.qlora_calib_stream_read(p, 1000, p, None) == -2                     # not a multiple of 16
    assert lib.qlora_calib_stream_read(ctypes.c_void_p((1 << 24) + 4), 1024, p, None) == -2  # misaligned
    assert lib.qlora_calib_stream_read(None, 1024, p, None) == -1


def test_adamw_host_errors(q):
    lib = q.raw()
    p = ctypes.c_void_p(1 << 24)
    f = ctypes.c_float
    assert lib.qlora_adamw_step(p, None, p, p, p, 0, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == 0      # empty
    assert lib.qlora_adamw_step(p, None, p, p, p, 16, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == -2    # step < 1
    assert lib.qlora_adamw_step(p, None, None, p, p, 16, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == -1
    assert lib.qlora_adamw_step(p, None, p, p, p, 16, 1, 1e-3, 1.0, 0.999, 1e-8, 0.0, None) == -1    # beta1 = 1
    assert lib.qlora_adamw_step(ctypes.c_void_p((1 << 24) + 4), None, p, p, p, 16, 1, 1e-3, 0.9, 0.999, 1e-8,
                                0.0, None) == -1                                                      # misaligned
    del f


def test_dropout_host_errors(q):
    """NULL or misaligned masks and keep scales below 1 are rejected before any
    launch; the dropout calls take the plain workspace."""
    lib = q.raw()
    W = _fake_weight(q)
    p = ctypes.c_void_p(1 << 24)
    big = 1 << 30
    assert lib.qlora_linear_fwd_dropout(ctypes.byref(W), p, 16, p, p, 8, 1.0, None, 1.05, p, None, p, big, None) == -1
    assert lib.qlora_linear_fwd_dropout(ctypes.byref(W), p, 16, p, p, 8, 1.0, ctypes.c_void_p((1 << 24) + 8), 1.05,
                                        p, None, p, big, None) == -1
    assert lib.qlora_linear_fwd_dropout(ctypes.byref(W), p, 16, p, p, 8, 1.0, p, 0.95, p, None, p, big, None) == -1
    assert lib.qlora_linear_fwd_dropout(ctypes.byref(W), p, 16, p, p, 8, 1.0, p, float("inf"), p, None, p, big,
                                        None) == -1
    assert lib.qlora_linear_bwd_dropout(ctypes.byref(W), p, None, p, 16, p, p, 8, 1.0, None, 1.05, p, p, p, 0, p,
                                        big, None) == -1
    # M = 0 succeeds without a mask check on shapes
    assert lib.qlora_linear_fwd_dropout(ctypes.byref(W), p, 0, p, p, 8, 1.0, p, 1.05, p, None, None, 0, None) == 0
    need = q.linear_workspace_bytes(64, 64, 128, 8, False)
    assert lib.qlora_linear_fwd_dropout(ctypes.byref(W), p, 64, p, p, 8, 1.0, p, 1.05, p, None, p, need - 1,
                                        None) == -4


def test_gemv_needs_its_workspace(q):
    lib = q.raw()
    W = _fake_weight(q)
    p = ctypes.c_void_p(1 << 24)
    need = q.nf4_gemv_workspace_bytes(128)
    assert need >= 16 * 128 * 2 and q.nf4_gemv_workspace_bytes(100) == 0
    assert lib.qlora_nf4_gemv_fwd(ctypes.byref(W), p, 4, p, p, 8, 1.0, p, None, 0, None) == -4
    assert lib.qlora_nf4_gemv_fwd(ctypes.byref(W), p, 4, p, p, 8, 1.0, p, p, need - 1, None) == -4
    assert lib.qlora_nf4_gemv_fwd(ctypes.byref(W), p, 17, p, p, 8, 1.0, p, p, need, None) == -2


def test_f16_host_checks(q):
    """The fp16 layer calls: their own workspace query, UNSUPPORTED for dX on an
    n that is not a multiple of 8, WORKSPACE before any launch, and the
    binding's dtype check."""
    lib = q.raw()
    W = _fake_weight(q, n=60)
    p = ctypes.c_void_p(1 << 24)
    big = 1 << 30
    # M <= 16 forward: GEMV workspace; M > 16: expanded path (expanded weight in it)
    assert q.linear_workspace_bytes(4, 60, 128, 8, False, torch.float16) >= q.nf4_gemv_workspace_bytes(128)
    assert q.linear_workspace_bytes(64, 64, 128, 8, False, torch.float16) >= 64 * 128 * 2
    assert q.linear_workspace_bytes(64, 60, 128, 8, True, torch.float16) > 0
    assert lib.qlora_linear_bwd_f16(ctypes.byref(W), p, None, p, 64, p, p, 8, 1.0, p, p, p, 0, p, big, None) == -3
    need = q.linear_workspace_bytes(64, 60, 128, 8, False, torch.float16)
    assert lib.qlora_linear_fwd_f16(ctypes.byref(W), p, 64, p, p, 8, 1.0, p, None, p, need - 1, None) == -4
    assert lib.qlora_linear_fwd_f16(ctypes.byref(W), p, 0, p, p, 8, 1.0, p, None, None, 0, None) == 0
    assert lib.qlora_dequant_f16(ctypes.byref(W), ctypes.c_void_p((1 << 24) + 8), None) == -1
    with pytest.raises(ValueError):
        q.linear_workspace_bytes(64, 64, 128, 8, False, torch.float32)


def test_dropout_in_fp16_is_rejected_before_any_call(q):
    """LoRA dropout exists in bf16 only: asking for it with the fp16 compute
    type raises on the host, in the forward as in the backward, before any
    tensor is checked or any library call is made."""
    cpu = torch.empty(0)
    w = q.NF4Weight(64, 128, cpu, cpu, cpu, cpu, cpu)
    X = torch.zeros((4, 128), dtype=torch.float16)
    mask = torch.ones((4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="bf16 only"):
        q.linear_fwd_dropout(w, X, None, None, 1.0, mask, 1.0, dtype=torch.float16)
    dY = torch.zeros((4, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="bf16 only"):
        q.linear_bwd_dropout(w, X, None, dY, None, None, 1.0, mask, 1.0, dtype=torch.float16)


def test_scratch_forward_refuses_oversize_before_any_call(q):
    """qlora_linear_fwd_scratch checks its need against the fixed scratch on
    the host and returns QLORA_ERR_SCRATCH before touching the device."""
    lib = q.raw()
    p = ctypes.c_void_p(1 << 24)
    base = 1 << 20
    w = q._Weight(8192, 8192, base, base + 4096, base + 8192, base + 12288, base + 16384, 0)
    assert q.linear_workspace_bytes(4096, 8192, 8192, 64, False) > q.SCRATCH_BYTES
    s = lib.qlora_linear_fwd_scratch(ctypes.byref(w), p, 4096, p, p, 64, 0.25, p, None, None)
    assert s == -6 and q.status_string(s).startswith("QLORA_ERR_SCRATCH")
    assert lib.qlora_linear_fwd_scratch(None, p, 4, p, p, 8, 1.0, p, None, None) == -1
    assert lib.qlora_linear_fwd_scratch(ctypes.byref(w), p, 4, p, p, 200, 1.0, p, None, None) == -2


def test_bf16_base_layer_argument_errors(q):
    """The bf16-base LoRA layer rejects k % 64 != 0 and bad ranks as SHAPE
    and NULL or misaligned pointers as INVALID_ARG, before any launch; M = 0
    with accumulate launches nothing."""
    lib = q.raw()
    p = ctypes.c_void_p(1 << 24)
    bad = ctypes.c_void_p((1 << 24) + 8)
    assert lib.qlora_lora_linear_fwd(p, 64, 100, p, 4, p, p, 8, 1.0, p, None, p, 1 << 20, None) == -2
    assert lib.qlora_lora_linear_fwd(p, 64, 128, p, 4, p, p, 200, 1.0, p, None, p, 1 << 20, None) == -2
    assert lib.qlora_lora_linear_fwd(None, 64, 128, p, 4, p, p, 8, 1.0, p, None, p, 1 << 20, None) == -1
    assert lib.qlora_lora_linear_fwd(bad, 64, 128, p, 4, p, p, 8, 1.0, p, None, p, 1 << 20, None) == -1
    assert lib.qlora_lora_linear_fwd(p, 64, 128, p, 4, p, p, 8, 1.0, p, None, p, 0, None) == -4
    assert lib.qlora_lora_linear_bwd(p, 64, 128, p, None, p, 0, p, p, 8, 1.0, p, p, p, 1, None, 0, None) == 0
    assert lib.qlora_lora_linear_workspace_bytes(4, 64, 100, 8, 0) == 0
    assert lib.qlora_lora_linear_workspace_bytes(4, 64, 128, 8, 1) > 0

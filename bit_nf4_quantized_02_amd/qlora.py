"""Thin Python binding over libqlora.so (ctypes).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every computation happens in the library's kernels.
Importing this module loads the library and raises ImportError if it has not
been built (``python -m bit_nf4_quantized_02_amd.build``) -- there is no
fallback of any kind.

Names follow the C ABI in include/qlora.h.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_nf4_quantized_02_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

BLOCK = 64
DQ_BLOCK = 256
MAX_RANK = 128
SCRATCH_BYTES = 64 << 20   # QLORA_SCRATCH_BYTES: the library's own device scratch per device
DT_BF16, DT_FP32 = 0, 1

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float


class _Weight(ctypes.Structure):
    _fields_ = [("n", _i64), ("k", _i64), ("codes", _vp), ("code8", _vp), ("s2", _vp), ("mean", _vp),
                ("codebook", _vp), ("scale_bf16", ctypes.c_int32)]


SCALE_FP32, SCALE_DQ, SCALE_BF16 = 0, 1, 2


_W = ctypes.POINTER(_Weight)

_SIGS = {
    "qlora_status_string": (ctypes.c_char_p, [_int]),
    "qlora_build_nf4_codebook": (_int, [ctypes.POINTER(_f)]),
    "qlora_nf4_packed_bytes": (_sz, [_i64, _i64]),
    "qlora_nf4_storage_bytes": (_sz, [_i64, _i64, _int]),
    "qlora_build_uniform4_codebook": (_int, [ctypes.POINTER(_f)]),
    "qlora_quantize_workspace_bytes": (_sz, [_i64, _i64]),
    "qlora_quantize_nf4": (_int, [_vp, _int, _W, _vp, _sz, _vp]),
    "qlora_dequant": (_int, [_W, _vp, _vp]),
    "qlora_linear_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int]),
    "qlora_linear_fwd": (_int, [_W, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _vp, _sz, _vp]),
    "qlora_linear_bwd": (_int, [_W, _vp, _vp, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _vp, _int, _vp, _sz, _vp]),
    "qlora_linear_fwd_scratch": (_int, [_W, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _vp]),
    "qlora_lora_linear_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int]),
    "qlora_lora_linear_fwd": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _vp, _sz, _vp]),
    "qlora_lora_linear_bwd": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _vp, _int,
                                      _vp, _sz, _vp]),
    "qlora_dequant_f16": (_int, [_W, _vp, _vp]),
    "qlora_linear_f16_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int]),
    "qlora_linear_fwd_f16": (_int, [_W, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _vp, _sz, _vp]),
    "qlora_linear_bwd_f16": (_int, [_W, _vp, _vp, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _vp, _int, _vp, _sz,
                                     _vp]),
    "qlora_linear_fwd_dropout": (_int, [_W, _vp, _i64, _vp, _vp, _int, _f, _vp, _f, _vp, _vp, _vp, _sz, _vp]),
    "qlora_linear_bwd_dropout": (_int, [_W, _vp, _vp, _vp, _i64, _vp, _vp, _int, _f, _vp, _f, _vp, _vp, _vp, _int,
                                         _vp, _sz, _vp]),
    "qlora_lowrank_split_cols": (_int, [_int]),
    "qlora_lowrank_project_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "qlora_lowrank_project": (_int, [_vp, _i64, _i64, _vp, _int, _int, _f, _vp, _vp, _vp, _sz, _vp]),
    "qlora_nf4_gemm_fwd": (_int, [_W, _vp, _i64, _vp, _vp, _int, _vp, _vp]),
    "qlora_nf4_gemm_dx": (_int, [_W, _vp, _i64, _vp, _vp, _int, _vp, _vp]),
    "qlora_nf4_gemv_fwd": (_int, [_W, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _sz, _vp]),
    "qlora_nf4_gemv_workspace_bytes": (_sz, [_i64]),
    "qlora_nf4_gemv_dx_workspace_bytes": (_sz, [_i64, _i64]),
    "qlora_nf4_gemv_dx": (_int, [_W, _vp, _i64, _vp, _vp, _int, _f, _vp, _vp, _sz, _vp]),
    "qlora_linear_path": (_int, [_i64, _i64, _i64, _int, _int]),
    "qlora_nf4_expand_bytes": (_sz, [_i64, _i64, _int, _int]),
    "qlora_nf4_expand": (_int, [_W, _vp, _int, _int, _vp, _sz, _vp]),
    "qlora_bf16_gemm_workspace_bytes": (_sz, [_i64, _i64, _int, _i64]),
    "qlora_bf16_gemm": (_int, [_vp, _i64, _i64, _vp, _int, _vp, _i64, _vp, _vp, _sz, _vp]),
    "qlora_bf16_gemm_nn": (_int, [_vp, _i64, _i64, _vp, _int, _vp, _i64, _vp, _vp, _sz, _vp]),
    "qlora_lowrank_grad_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "qlora_lowrank_grad": (_int, [_vp, _i64, _i64, _vp, _int, _f, _vp, _int, _int, _vp, _sz, _vp]),
    "qlora_silu_mul_fwd": (_int, [_vp, _vp, _vp, _i64, _vp]),
    "qlora_silu_mul_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "qlora_adapter_merge": (_int, [_W, _vp, _vp, _int, _f, _vp, _int, _vp]),
    "qlora_adapter_unmerge": (_int, [_vp, _i64, _i64, _vp, _vp, _int, _f, _vp, _vp]),
    "qlora_adamw_step": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _f, _f, _f, _f, _f, _vp]),
    "qlora_calib_mfma": (_int, [_int, _int, _vp, _vp]),
    "qlora_calib_stream_read": (_int, [_vp, _i64, _vp, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class QLoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


def status_string(status: int) -> str:
    return _lib.qlora_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise QLoraError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} device={t.device}")


def _bytes(nbytes: int, device) -> torch.Tensor | None:
    return torch.empty(max(int(nbytes), 0), dtype=torch.uint8, device=device) if nbytes > 0 else None


# --------------------------------------------------------------------------- codebook

def build_nf4_codebook() -> list[float]:
    """The 16 NF4 levels (host, fp32), ascending."""
    buf = (_f * 16)()
    _check(_lib.qlora_build_nf4_codebook(buf), "qlora_build_nf4_codebook")
    return [buf[i] for i in range(16)]


def build_uniform4_codebook() -> list[float]:
    """The 16 levels of the uniform INT4 grid (host, fp32), ascending."""
    buf = (_f * 16)()
    _check(_lib.qlora_build_uniform4_codebook(buf), "qlora_build_uniform4_codebook")
    return [buf[i] for i in range(16)]


def nf4_packed_bytes(n: int, k: int, double_quant: bool = True, scale_dtype=torch.float32) -> int:
    """Bytes of an encoded weight; without double quantization the block
    scales are fp32, or bf16 with scale_dtype=torch.bfloat16."""
    form = SCALE_DQ if double_quant else (SCALE_BF16 if scale_dtype == torch.bfloat16 else SCALE_FP32)
    return int(_lib.qlora_nf4_storage_bytes(n, k, form))


def quantize_workspace_bytes(n: int, k: int) -> int:
    return int(_lib.qlora_quantize_workspace_bytes(n, k))


def linear_workspace_bytes(M: int, n: int, k: int, r: int, is_bwd: bool, dtype=torch.bfloat16) -> int:
    fn = _lib.qlora_linear_f16_workspace_bytes if _is_f16(dtype) else _lib.qlora_linear_workspace_bytes
    return int(fn(M, n, k, r, int(bool(is_bwd))))


def _is_f16(dtype) -> bool:
    """The 16-bit compute type of a layer call: bf16 (default) or fp16."""
    if dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"compute dtype must be torch.bfloat16 or torch.float16, got {dtype}")
    return dtype == torch.float16


# --------------------------------------------------------------------------- weight

@dataclass
class NF4Weight:
    """Device buffers of one encoded [n, k] weight (owned by these tensors)."""
    n: int
    k: int
    codes: torch.Tensor      # uint8 [n, k/2]
    code8: torch.Tensor | None   # uint8 [n*k/64] (None: no double quantization)
    s2: torch.Tensor             # fp32  [ceil(nb/256)], or [nb] fp32 / bf16 block scales without it
    mean: torch.Tensor | None    # fp32  [1]
    codebook: torch.Tensor   # fp32  [16]

    @staticmethod
    def empty(n: int, k: int, device="cuda", codebook: torch.Tensor | None = None,
              double_quant: bool = True, scale_dtype=torch.float32) -> "NF4Weight":
        """Buffers for one encoded weight; without double quantization code8
        and mean are None and s2 holds one scale per block, fp32 or (with
        scale_dtype=torch.bfloat16) bf16."""
        nb = n * k // BLOCK
        nc = -(-nb // DQ_BLOCK)
        if codebook is None:
            codebook = torch.tensor(build_nf4_codebook(), dtype=torch.float32, device=device)
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=device)
        if not double_quant:
            if scale_dtype not in (torch.float32, torch.bfloat16):
                raise ValueError("block scales are fp32 or bf16")
            return NF4Weight(n, k, codes, None, torch.empty((nb,), dtype=scale_dtype, device=device), None,
                             codebook)
        if scale_dtype != torch.float32:
            raise ValueError("a bf16 block scale is a form without double quantization")
        return NF4Weight(n, k, codes,
                         torch.empty((nb,), dtype=torch.uint8, device=device),
                         torch.empty((nc,), dtype=torch.float32, device=device),
                         torch.empty((1,), dtype=torch.float32, device=device),
                         codebook)

    @property
    def double_quant(self) -> bool:
        return self.code8 is not None

    @property
    def scale_bf16(self) -> bool:
        return self.code8 is None and self.s2.dtype == torch.bfloat16

    def struct(self) -> _Weight:
        p = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        return _Weight(self.n, self.k, self.codes.data_ptr(), p(self.code8), self.s2.data_ptr(),
                       p(self.mean), self.codebook.data_ptr(), int(self.scale_bf16))

    def nbytes(self) -> int:
        return nf4_packed_bytes(self.n, self.k, self.double_quant,
                                torch.bfloat16 if self.scale_bf16 else torch.float32)


def quantize_nf4(W: torch.Tensor, out: NF4Weight | None = None, ws: torch.Tensor | None = None,
                 stream=None, codebook: torch.Tensor | None = None, double_quant: bool = True,
                 scale_dtype=torch.float32) -> NF4Weight:
    """Encode W ([n, k] bf16 or fp32, on the GPU) as 4-bit codes + block
    scales, double-quantized unless double_quant is False (then one fp32, or
    with scale_dtype=torch.bfloat16 one bf16, scale per block); the levels
    are NF4 unless another 16-level device codebook is given (or out's)."""
    if W.dim() != 2:
        raise ValueError("W must be [n, k]")
    n, k = W.shape
    dt = {torch.bfloat16: DT_BF16, torch.float32: DT_FP32}.get(W.dtype)
    if dt is None:
        raise ValueError("W must be bf16 or fp32")
    _need(W, W.dtype, (n, k), "W")
    if out is None:
        out = NF4Weight.empty(n, k, device=W.device, codebook=codebook, double_quant=double_quant,
                              scale_dtype=scale_dtype)
    need = quantize_workspace_bytes(n, k)
    if ws is None:
        ws = _bytes(need, W.device)
    st = out.struct()
    _check(_lib.qlora_quantize_nf4(_ptr(W), dt, ctypes.byref(st), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(stream)), "qlora_quantize_nf4")
    return out


def dequant(w: NF4Weight, out: torch.Tensor | None = None, stream=None, dtype=torch.bfloat16) -> torch.Tensor:
    """[n, k] expansion in bf16 (or fp16), bit-identical to what the GEMM kernels multiply."""
    f16 = _is_f16(dtype)
    if out is None:
        out = torch.empty((w.n, w.k), dtype=dtype, device=w.codes.device)
    _need(out, dtype, (w.n, w.k), "out")
    st = w.struct()
    name = "qlora_dequant_f16" if f16 else "qlora_dequant"
    _check(getattr(_lib, name)(ctypes.byref(st), _ptr(out), _stream(stream)), name)
    return out


# --------------------------------------------------------------------------- linear

def _mask_of(mask: torch.Tensor, M: int, k: int):
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (M, k) or not mask.is_contiguous() or not mask.is_cuda:
        raise ValueError(f"mask: expected contiguous uint8 {(M, k)} on the GPU")
    return _ptr(mask)


def linear_fwd_dropout(w: NF4Weight, X: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None, scale: float,
                       mask: torch.Tensor, keep_scale: float, **kw):
    """Y = X W'^T + scale ((X . mask * keep_scale) A^T) B^T (qlora_linear_fwd_dropout);
    the saved T is (X . mask) A^T.  Returns (Y, T)."""
    return linear_fwd(w, X, A, B, scale, _dropout=(mask, keep_scale), **kw)


def linear_bwd_dropout(w: NF4Weight, X: torch.Tensor | None, T: torch.Tensor | None, dY: torch.Tensor,
                       A: torch.Tensor | None, B: torch.Tensor | None, scale: float, mask: torch.Tensor,
                       keep_scale: float, **kw):
    """The gradients of linear_fwd_dropout (qlora_linear_bwd_dropout).  Returns (dX, dA, dB)."""
    return linear_bwd(w, X, T, dY, A, B, scale, _dropout=(mask, keep_scale), **kw)


def linear_fwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None, scale: float,
               Y: torch.Tensor | None = None, T: torch.Tensor | None = None, save_T: bool = True,
               ws: torch.Tensor | None = None, stream=None, _dropout=None, dtype=torch.bfloat16):
    """Y = X W'^T + scale (X A^T) B^T.  Returns (Y, T) with T None unless saved.
    dtype=torch.float16 runs the fp16 layer (qlora_linear_fwd_f16)."""
    M = X.shape[0]
    r = 0 if A is None else A.shape[0]
    f16 = _is_f16(dtype)
    if f16 and _dropout is not None:
        raise ValueError("LoRA dropout runs in bf16 only")
    _need(X, dtype, (M, w.k), "X")
    if r:
        _need(A, dtype, (r, w.k), "A")
        _need(B, dtype, (w.n, r), "B")
    if Y is None:
        Y = torch.empty((M, w.n), dtype=dtype, device=X.device)
    _need(Y, dtype, (M, w.n), "Y")
    if T is None and save_T and r:
        T = torch.empty((M, r), dtype=torch.float32, device=X.device)
    if T is not None:
        _need(T, torch.float32, (M, r), "T")
    st = w.struct()
    if _dropout is not None:
        mp = _mask_of(_dropout[0], M, w.k)
        if ws is None:
            ws = _bytes(linear_workspace_bytes(M, w.n, w.k, r, False), X.device)
        _check(_lib.qlora_linear_fwd_dropout(ctypes.byref(st), _ptr(X), M, _ptr(A), _ptr(B), r, float(scale), mp,
                                             float(_dropout[1]), _ptr(Y), _ptr(T), _ptr(ws),
                                             0 if ws is None else ws.numel(), _stream(stream)),
               "qlora_linear_fwd_dropout")
        return Y, T
    if ws is None:
        ws = _bytes(linear_workspace_bytes(M, w.n, w.k, r, False, dtype), X.device)
    name = "qlora_linear_fwd_f16" if f16 else "qlora_linear_fwd"
    _check(getattr(_lib, name)(ctypes.byref(st), _ptr(X), M, _ptr(A), _ptr(B), r, float(scale), _ptr(Y), _ptr(T),
                               _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), name)
    return Y, T


def linear_fwd_scratch(w: NF4Weight, X: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None,
                       scale: float, Y: torch.Tensor | None = None, T: torch.Tensor | None = None,
                       save_T: bool = True, stream=None):
    """linear_fwd with no workspace (qlora_linear_fwd_scratch): the library's
    own device scratch serves instead, so the call allocates nothing when Y
    (and T, if saved) are given. Calls overlapping on one device race.
    Returns (Y, T)."""
    M = X.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(X, torch.bfloat16, (M, w.k), "X")
    if r:
        _need(A, torch.bfloat16, (r, w.k), "A")
        _need(B, torch.bfloat16, (w.n, r), "B")
    if Y is None:
        Y = torch.empty((M, w.n), dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, (M, w.n), "Y")
    if T is None and save_T and r:
        T = torch.empty((M, r), dtype=torch.float32, device=X.device)
    if T is not None:
        _need(T, torch.float32, (M, r), "T")
    st = w.struct()
    _check(_lib.qlora_linear_fwd_scratch(ctypes.byref(st), _ptr(X), M, _ptr(A), _ptr(B), r, float(scale), _ptr(Y),
                                         _ptr(T), _stream(stream)), "qlora_linear_fwd_scratch")
    return Y, T


def linear_bwd(w: NF4Weight, X: torch.Tensor | None, T: torch.Tensor | None, dY: torch.Tensor,
               A: torch.Tensor | None, B: torch.Tensor | None, scale: float, need_dX: bool = True,
               need_dA: bool = True, need_dB: bool = True, dX: torch.Tensor | None = None,
               dA: torch.Tensor | None = None, dB: torch.Tensor | None = None, accumulate: bool = False,
               ws: torch.Tensor | None = None, stream=None, _dropout=None, dtype=torch.bfloat16):
    """dX = dY W' + s (dY B) A;  dA = s (dY B)^T X;  dB = s dY^T T.  Returns (dX, dA, dB).
    dtype=torch.float16 runs the fp16 layer (qlora_linear_bwd_f16)."""
    M = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    dev = dY.device
    f16 = _is_f16(dtype)
    if f16 and _dropout is not None:
        raise ValueError("LoRA dropout runs in bf16 only")
    _need(dY, dtype, (M, w.n), "dY")
    if X is not None:
        _need(X, dtype, (M, w.k), "X")
    if r:
        _need(A, dtype, (r, w.k), "A")
        _need(B, dtype, (w.n, r), "B")
    if T is not None:
        _need(T, torch.float32, (M, r), "T")
    if need_dX and dX is None:
        dX = torch.empty((M, w.k), dtype=dtype, device=dev)
    if r and need_dA and dA is None:
        dA = (torch.zeros if accumulate else torch.empty)((r, w.k), dtype=torch.float32, device=dev)
    if r and need_dB and dB is None:
        dB = (torch.zeros if accumulate else torch.empty)((w.n, r), dtype=torch.float32, device=dev)
    if dX is not None:
        _need(dX, dtype, (M, w.k), "dX")
    if dA is not None:
        _need(dA, torch.float32, (r, w.k), "dA")
    if dB is not None:
        _need(dB, torch.float32, (w.n, r), "dB")
    st = w.struct()
    if _dropout is not None:
        mp = _mask_of(_dropout[0], M, w.k)
        if ws is None:
            ws = _bytes(linear_workspace_bytes(M, w.n, w.k, r, True), dev)
        _check(_lib.qlora_linear_bwd_dropout(ctypes.byref(st), _ptr(X), _ptr(T), _ptr(dY), M, _ptr(A), _ptr(B), r,
                                             float(scale), mp, float(_dropout[1]), _ptr(dX), _ptr(dA), _ptr(dB),
                                             int(bool(accumulate)), _ptr(ws), 0 if ws is None else ws.numel(),
                                             _stream(stream)), "qlora_linear_bwd_dropout")
        return dX, dA, dB
    if ws is None:
        ws = _bytes(linear_workspace_bytes(M, w.n, w.k, r, True, dtype), dev)
    name = "qlora_linear_bwd_f16" if f16 else "qlora_linear_bwd"
    _check(getattr(_lib, name)(ctypes.byref(st), _ptr(X), _ptr(T), _ptr(dY), M, _ptr(A), _ptr(B), r, float(scale),
                               _ptr(dX), _ptr(dA), _ptr(dB), int(bool(accumulate)), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(stream)), name)
    return dX, dA, dB


# --------------------------------------------------------------------------- bf16-base LoRA layer

def lora_linear_workspace_bytes(M: int, n: int, k: int, r: int, is_bwd: bool) -> int:
    return int(_lib.qlora_lora_linear_workspace_bytes(M, n, k, r, int(bool(is_bwd))))


def lora_linear_fwd(W: torch.Tensor, X: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None, scale: float,
                    Y: torch.Tensor | None = None, T: torch.Tensor | None = None, save_T: bool = True,
                    ws: torch.Tensor | None = None, stream=None):
    """Y = X W^T + scale (X A^T) B^T over a bf16 base W [n, k]
    (qlora_lora_linear_fwd).  Returns (Y, T)."""
    n, k = W.shape
    M = X.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(W, torch.bfloat16, (n, k), "W")
    _need(X, torch.bfloat16, (M, k), "X")
    if r:
        _need(A, torch.bfloat16, (r, k), "A")
        _need(B, torch.bfloat16, (n, r), "B")
    if Y is None:
        Y = torch.empty((M, n), dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, (M, n), "Y")
    if T is None and save_T and r:
        T = torch.empty((M, r), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = _bytes(lora_linear_workspace_bytes(M, n, k, r, False), X.device)
    _check(_lib.qlora_lora_linear_fwd(_ptr(W), n, k, _ptr(X), M, _ptr(A), _ptr(B), r, float(scale), _ptr(Y), _ptr(T),
                                      _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "qlora_lora_linear_fwd")
    return Y, T


def lora_linear_bwd(W: torch.Tensor, X: torch.Tensor | None, T: torch.Tensor | None, dY: torch.Tensor,
                    A: torch.Tensor | None, B: torch.Tensor | None, scale: float, need_dX: bool = True,
                    need_dA: bool = True, need_dB: bool = True, accumulate: bool = False,
                    ws: torch.Tensor | None = None, stream=None):
    """The gradients of lora_linear_fwd (qlora_lora_linear_bwd).  Returns (dX, dA, dB)."""
    n, k = W.shape
    M = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    dev = dY.device
    _need(W, torch.bfloat16, (n, k), "W")
    _need(dY, torch.bfloat16, (M, n), "dY")
    if X is not None:
        _need(X, torch.bfloat16, (M, k), "X")
    if r:
        _need(A, torch.bfloat16, (r, k), "A")
        _need(B, torch.bfloat16, (n, r), "B")
    if T is not None:
        _need(T, torch.float32, (M, r), "T")
    dX = torch.empty((M, k), dtype=torch.bfloat16, device=dev) if need_dX else None
    mk = torch.zeros if accumulate else torch.empty
    dA = mk((r, k), dtype=torch.float32, device=dev) if (r and need_dA) else None
    dB = mk((n, r), dtype=torch.float32, device=dev) if (r and need_dB) else None
    if ws is None:
        ws = _bytes(lora_linear_workspace_bytes(M, n, k, r, True), dev)
    _check(_lib.qlora_lora_linear_bwd(_ptr(W), n, k, _ptr(X), _ptr(T), _ptr(dY), M, _ptr(A), _ptr(B), r, float(scale),
                                      _ptr(dX), _ptr(dA), _ptr(dB), int(bool(accumulate)), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(stream)), "qlora_lora_linear_bwd")
    return dX, dA, dB


# --------------------------------------------------------------------------- building blocks

def lowrank_split_cols(r: int) -> int:
    return int(_lib.qlora_lowrank_split_cols(r))


def lowrank_project(P: torch.Tensor, Q: torch.Tensor, q_layout: int, scale: float, want_out: bool = True,
                    want_split: bool = False, out: torch.Tensor | None = None, split: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None, stream=None):
    """out = P Q^T (q_layout 0, Q [r, C]) or P Q (q_layout 1, Q [C, r]), fp32; split = bf16 hi/lo of scale*out."""
    M, C = P.shape
    r = Q.shape[0] if q_layout == 0 else Q.shape[1]
    _need(P, torch.bfloat16, (M, C), "P")
    _need(Q, torch.bfloat16, (r, C) if q_layout == 0 else (C, r), "Q")
    if want_out and out is None:
        out = torch.empty((M, r), dtype=torch.float32, device=P.device)
    if want_split and split is None:
        split = torch.empty((M, lowrank_split_cols(r)), dtype=torch.bfloat16, device=P.device)
    if ws is None:
        ws = _bytes(int(_lib.qlora_lowrank_project_workspace_bytes(M, C, r)), P.device)
    _check(_lib.qlora_lowrank_project(_ptr(P), M, C, _ptr(Q), int(q_layout), r, float(scale), _ptr(out), _ptr(split),
                                      _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "qlora_lowrank_project")
    return out, split


def nf4_gemm_fwd(w: NF4Weight, X: torch.Tensor, split: torch.Tensor | None, B: torch.Tensor | None,
                 Y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    M = X.shape[0]
    r = 0 if B is None else B.shape[1]
    if Y is None:
        Y = torch.empty((M, w.n), dtype=torch.bfloat16, device=X.device)
    st = w.struct()
    _check(_lib.qlora_nf4_gemm_fwd(ctypes.byref(st), _ptr(X), M, _ptr(split), _ptr(B), r, _ptr(Y), _stream(stream)),
           "qlora_nf4_gemm_fwd")
    return Y


def nf4_gemm_dx(w: NF4Weight, dY: torch.Tensor, split: torch.Tensor | None, A: torch.Tensor | None,
                dX: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    M = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    if dX is None:
        dX = torch.empty((M, w.k), dtype=torch.bfloat16, device=dY.device)
    st = w.struct()
    _check(_lib.qlora_nf4_gemm_dx(ctypes.byref(st), _ptr(dY), M, _ptr(split), _ptr(A), r, _ptr(dX), _stream(stream)),
           "qlora_nf4_gemm_dx")
    return dX


PATH_GEMV, PATH_FUSED, PATH_EXPANDED = 0, 1, 2


def linear_path(M: int, n: int, k: int, r: int, is_bwd: bool) -> int:
    p = _lib.qlora_linear_path(M, n, k, r, int(is_bwd))
    if p < 0:
        raise QLoraError(-1, "qlora_linear_path")
    return p


def nf4_expand_bytes(n: int, k: int, r: int, transposed: int) -> int:
    return int(_lib.qlora_nf4_expand_bytes(n, k, r, int(transposed)))


def nf4_expand(w: NF4Weight, lr: torch.Tensor | None, r: int, transposed: int, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """Expanded bf16 operand: [n, k + xc] (transposed = 0, forward, lr = B),
    [k, np + xc] (1, for dX, lr = A) or [n + xc, k] (2, contraction-major for
    dX, n % 64 == 0, lr = A); returned as a 2-D bf16 tensor."""
    xc = lowrank_split_cols(r)
    transposed = int(transposed)
    if transposed == 1:
        rows, cols = w.k, ((w.n + 63) // 64) * 64 + xc
    elif transposed == 2:
        rows, cols = w.n + xc, w.k
    else:
        rows, cols = w.n, w.k + xc
    nbytes = nf4_expand_bytes(w.n, w.k, r, transposed)
    if out is None:
        out = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.codes.device)
    st = w.struct()
    _check(_lib.qlora_nf4_expand(ctypes.byref(st), _ptr(lr), r, int(transposed), _ptr(out), out.numel() * 2,
                                 _stream(stream)), "qlora_nf4_expand")
    return out.view(-1)[: rows * cols].view(rows, cols)


def bf16_gemm_nn(act: torch.Tensor, split: torch.Tensor | None, r: int, F: torch.Tensor, nout: int,
                 out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out = RN_bf16(act F[:kc] + split F[kc:]) over the contraction-major
    operand of nf4_expand(..., transposed=2)."""
    M, kc = act.shape
    if out is None:
        out = torch.empty((M, nout), dtype=torch.bfloat16, device=act.device)
    if ws is None:
        ws = _bytes(bf16_gemm_workspace_bytes(M, kc, r, nout), act.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.qlora_bf16_gemm_nn(_ptr(act), M, kc, _ptr(split), r, _ptr(F), nout, _ptr(out), _ptr(ws), nbytes,
                                   _stream(stream)), "qlora_bf16_gemm_nn")
    return out


def bf16_gemm_workspace_bytes(M: int, kc: int, r: int, nout: int) -> int:
    return int(_lib.qlora_bf16_gemm_workspace_bytes(M, kc, r, nout))


def bf16_gemm(act: torch.Tensor, split: torch.Tensor | None, r: int, F: torch.Tensor, nout: int,
              out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    M, kc = act.shape
    if out is None:
        out = torch.empty((M, nout), dtype=torch.bfloat16, device=act.device)
    if ws is None:
        ws = _bytes(bf16_gemm_workspace_bytes(M, kc, r, nout), act.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.qlora_bf16_gemm(_ptr(act), M, kc, _ptr(split), r, _ptr(F), nout, _ptr(out), _ptr(ws), nbytes,
                                _stream(stream)), "qlora_bf16_gemm")
    return out


def nf4_gemv_workspace_bytes(k: int) -> int:
    return int(_lib.qlora_nf4_gemv_workspace_bytes(k))


def nf4_gemv_fwd(w: NF4Weight, X: torch.Tensor, T: torch.Tensor | None, B: torch.Tensor | None, scale: float,
                 Y: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    M = X.shape[0]
    r = 0 if B is None else B.shape[1]
    if Y is None:
        Y = torch.empty((M, w.n), dtype=torch.bfloat16, device=X.device)
    if ws is None:
        ws = _bytes(nf4_gemv_workspace_bytes(w.k), X.device)
    st = w.struct()
    _check(_lib.qlora_nf4_gemv_fwd(ctypes.byref(st), _ptr(X), M, _ptr(T), _ptr(B), r, float(scale), _ptr(Y),
                                   _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "qlora_nf4_gemv_fwd")
    return Y


def nf4_gemv_dx_workspace_bytes(n: int, k: int) -> int:
    return int(_lib.qlora_nf4_gemv_dx_workspace_bytes(n, k))


def nf4_gemv_dx(w: NF4Weight, dY: torch.Tensor, U: torch.Tensor | None, A: torch.Tensor | None, scale: float,
                dX: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """dX = dY W' + scale U A for M <= 16 (qlora_nf4_gemv_dx); U = dY B fp32."""
    M = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    if dX is None:
        dX = torch.empty((M, w.k), dtype=torch.bfloat16, device=dY.device)
    if ws is None:
        ws = _bytes(nf4_gemv_dx_workspace_bytes(w.n, w.k), dY.device)
    st = w.struct()
    _check(_lib.qlora_nf4_gemv_dx(ctypes.byref(st), _ptr(dY), M, _ptr(U), _ptr(A), r, float(scale), _ptr(dX),
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "qlora_nf4_gemv_dx")
    return dX


def lowrank_grad(P: torch.Tensor, Q: torch.Tensor, scale: float, g_layout: int, G: torch.Tensor | None = None,
                 accumulate: bool = False, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """G = scale P^T Q as [r, C] (g_layout 0) or [C, r] (g_layout 1), fp32."""
    M, C = P.shape
    r = Q.shape[1]
    if G is None:
        G = (torch.zeros if accumulate else torch.empty)((r, C) if g_layout == 0 else (C, r), dtype=torch.float32,
                                                         device=P.device)
    if ws is None:
        ws = _bytes(int(_lib.qlora_lowrank_grad_workspace_bytes(M, C, r)), P.device)
    _check(_lib.qlora_lowrank_grad(_ptr(P), M, C, _ptr(Q), r, float(scale), _ptr(G), int(g_layout),
                                   int(bool(accumulate)), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "qlora_lowrank_grad")
    return G


class Call:
    """One C-ABI call with its ctypes arguments prebuilt (for tight timing
    loops); calling it only forwards the stored arguments."""

    def __init__(self, name: str, *args, keep=()):
        self.name = name
        self.fn = getattr(_lib, name)
        self.args = args
        self._keep = keep  # keeps ctypes structs referenced by pointer alive

    def __call__(self):
        s = self.fn(*self.args)
        if s != 0:
            raise QLoraError(s, self.name)


# --------------------------------------------------------------------------- MLP join

def silu_mul_fwd(G: torch.Tensor, U: torch.Tensor, H: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _need(U, torch.bfloat16, G.shape, "Up")
    _need(G, torch.bfloat16, G.shape, "G")
    if H is None:
        H = torch.empty_like(G)
    _check(_lib.qlora_silu_mul_fwd(_ptr(G), _ptr(U), _ptr(H), G.numel(), _stream(stream)), "qlora_silu_mul_fwd")
    return H


def silu_mul_bwd(G: torch.Tensor, U: torch.Tensor, dH: torch.Tensor, stream=None):
    for t, nme in ((G, "G"), (U, "Up"), (dH, "dH")):
        _need(t, torch.bfloat16, G.shape, nme)
    dG = torch.empty_like(G)
    dU = torch.empty_like(G)
    _check(_lib.qlora_silu_mul_bwd(_ptr(G), _ptr(U), _ptr(dH), _ptr(dG), _ptr(dU), G.numel(), _stream(stream)),
           "qlora_silu_mul_bwd")
    return dG, dU


def adapter_merge(w: NF4Weight, A: torch.Tensor | None, B: torch.Tensor | None, scale: float,
                  out_dtype=torch.bfloat16, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """round(W' + scale * B A) as a [n, k] bf16 or fp32 tensor."""
    r = 0 if A is None else A.shape[0]
    if r:
        _need(A, torch.bfloat16, (r, w.k), "A")
        _need(B, torch.bfloat16, (w.n, r), "B")
    dt = {torch.bfloat16: 0, torch.float32: 1}[out_dtype]
    if out is None:
        out = torch.empty((w.n, w.k), dtype=out_dtype, device=w.codes.device)
    _need(out, out_dtype, (w.n, w.k), "out")
    st = w.struct()
    _check(_lib.qlora_adapter_merge(ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale), _ptr(out), dt,
                                    _stream(stream)), "qlora_adapter_merge")
    return out


def adapter_unmerge(merged: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None, scale: float,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """RN_bf16(merged - scale * B A); out may be `merged` itself."""
    n, k = merged.shape
    r = 0 if A is None else A.shape[0]
    _need(merged, torch.bfloat16, (n, k), "merged")
    if r:
        _need(A, torch.bfloat16, (r, k), "A")
        _need(B, torch.bfloat16, (n, r), "B")
    if out is None:
        out = torch.empty_like(merged)
    _check(_lib.qlora_adapter_unmerge(_ptr(merged), n, k, _ptr(A), _ptr(B), r, float(scale), _ptr(out),
                                      _stream(stream)), "qlora_adapter_unmerge")
    return out


def adamw_step(theta: torch.Tensor, grad: torch.Tensor, m: torch.Tensor, v: torch.Tensor, step: int, lr: float,
               betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0,
               theta16: torch.Tensor | None = None, stream=None) -> None:
    """In-place AdamW step; m and v may be CPU tensors in pinned memory."""
    n = theta.numel()
    for t, nme in ((theta, "theta"), (grad, "grad")):
        _need(t, torch.float32, theta.shape, nme)
    for t, nme in ((m, "m"), (v, "v")):
        if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{nme}: expected contiguous fp32 with {n} elements on the GPU or in pinned host memory")
    if theta16 is not None:
        _need(theta16, torch.bfloat16, theta.shape, "theta16")
    _check(_lib.qlora_adamw_step(_ptr(theta), _ptr(theta16), _ptr(grad), ctypes.c_void_p(m.data_ptr()),
                                 ctypes.c_void_p(v.data_ptr()), n, int(step), float(lr), float(betas[0]),
                                 float(betas[1]), float(eps), float(weight_decay), _stream(stream)),
           "qlora_adamw_step")


def calib_mfma(blocks: int, iters: int, sink: torch.Tensor, stream=None) -> int:
    """Enqueue the matrix-core probe; returns its flop count."""
    _need(sink, torch.float32, sink.shape, "sink")
    _check(_lib.qlora_calib_mfma(blocks, iters, _ptr(sink), _stream(stream)), "qlora_calib_mfma")
    return blocks * 8 * iters * 8 * 32768


def calib_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> int:
    """Enqueue one streaming read of `buf`; returns the bytes read."""
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.qlora_calib_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "qlora_calib_stream_read")
    return nbytes


def raw():
    """The ctypes handle, for tests that call the C ABI directly."""
    return _lib

"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and holds the workload shapes; it
contains none of the method's arithmetic (no quantization, no scale, no
product), so both the HIP path and the CPU oracle can be fed from it without
sharing code.

Recipe (the pages name no dataset; these shapes stand in for the 7B / 65B /
70B-class linears that "QLoRA Explained ..." (gamut.so) tabulates in
"QLoRA vs LoRA: Memory, Speed, and Quality Tradeoffs"):
  W  ~ N(0, sigma) drawn in fp32 then rounded to bf16 (RNE); optionally a
       seeded set of exactly round(frac * N * K) distinct positions is
       multiplied by 10 before the rounding (outliers);
  X, dY ~ N(0, 1) -> bf16;
  A  ~ U(-1/sqrt(K), +1/sqrt(K)) -> bf16 (Kaiming-uniform with a = sqrt 5);
  B  ~ N(0, 0.01) -> bf16.
Host draws use numpy's PCG64 seeded with the tuple (config, layer, tensor);
the 65B stack's layers past the first draw W, A, B on the device instead
(torch's Philox generator, same distributions and seed tuples).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

T_W, T_X, T_A, T_B, T_DY, T_MASK = 0, 1, 2, 3, 4, 5


def rng(*seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))


def to_bf16(a32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)


def normal_bf16(shape, std: float, *seed: int) -> torch.Tensor:
    g = rng(*seed)
    return to_bf16(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


def uniform_bf16(shape, bound: float, *seed: int) -> torch.Tensor:
    g = rng(*seed)
    return to_bf16(g.uniform(-bound, bound, size=shape).astype(np.float32))


def weight_bf16(n: int, k: int, sigma: float, *seed: int, outlier_frac: float = 0.0) -> torch.Tensor:
    g = rng(*seed)
    w = g.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)
    if outlier_frac > 0.0:
        cnt = int(round(outlier_frac * n * k))
        pos = g.choice(n * k, size=cnt, replace=False)
        w.reshape(-1)[pos] *= np.float32(10.0)
    return to_bf16(w)


def device_seed(*seed: int) -> int:
    """One 63-bit integer from the seed tuple, for torch's device generator."""
    return int(np.random.SeedSequence(list(seed)).generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def device_normal_bf16(shape, std: float, *seed: int, device: str = "cuda") -> torch.Tensor:
    """N(0, std) drawn on the device with torch's Philox generator seeded
    from the tuple, in fp32, then rounded to bf16 (RNE): for workloads too
    large to draw on the host (the 65B stack's weights). Not the same numbers
    as the host draw of the same tuple."""
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(*seed))
    w = torch.empty(shape, dtype=torch.float32, device=device)
    w.normal_(0.0, std, generator=g)
    return w.to(torch.bfloat16)


def device_uniform_bf16(shape, bound: float, *seed: int, device: str = "cuda") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(*seed))
    w = torch.empty(shape, dtype=torch.float32, device=device)
    w.uniform_(-bound, bound, generator=g)
    return w.to(torch.bfloat16)


def dropout_mask(m: int, k: int, p: float, *seed: int) -> torch.Tensor:
    """uint8 [m, k] keep mask of the adapter-input dropout: 1 with probability
    1 - p, else 0 (the caller draws it; kernels only read it)."""
    g = rng(*seed)
    return torch.from_numpy((g.random((m, k)) >= p).astype(np.uint8))


def lora_A(r: int, k: int, *seed: int) -> torch.Tensor:
    return uniform_bf16((r, k), 1.0 / math.sqrt(k), *seed)


def lora_B(n: int, r: int, *seed: int) -> torch.Tensor:
    return normal_bf16((n, r), 0.01, *seed)


@dataclass
class Linear:
    name: str
    n: int   # out features
    k: int   # in features


@dataclass
class Config:
    cid: int
    title: str
    linears: list
    m: list            # token counts
    r: int
    alpha: float
    sigma: float
    outlier_frac: float = 0.0
    layers: int = 1
    backward: bool = True
    chain_silu: bool = False

    @property
    def scale(self) -> float:
        return self.alpha / self.r if self.r > 0 else 0.0


CONFIGS = {
    1: Config(1, "single 1024x1024 QLoRA linear, M=16",
              [Linear("w", 1024, 1024)], [16], r=8, alpha=16, sigma=0.02),
    2: Config(2, "7B-class attention projection 4096x4096, M=4096",
              [Linear("proj", 4096, 4096)], [4096], r=16, alpha=32, sigma=0.02),
    3: Config(3, "7B-class MLP gate/up 4096->11008, down 11008->4096, M=2048",
              [Linear("gate", 11008, 4096), Linear("up", 11008, 4096), Linear("down", 4096, 11008)],
              [2048], r=64, alpha=16, sigma=0.02, outlier_frac=0.001, chain_silu=True),
    4: Config(4, "70B-class MLP decode GEMV 8192<->28672, M in {1,4,16}",
              [Linear("up", 28672, 8192), Linear("down", 8192, 28672)],
              [1, 4, 16], r=16, alpha=16, sigma=0.015, backward=False),
    5: Config(5, "65B-class stack, 80 layers x (q,k,v,o 8192x8192; gate,up 8192->22016; down 22016->8192), M=4096",
              [Linear("q", 8192, 8192), Linear("k", 8192, 8192), Linear("v", 8192, 8192),
               Linear("o", 8192, 8192), Linear("gate", 22016, 8192), Linear("up", 22016, 8192),
               Linear("down", 8192, 22016)],
              [4096], r=64, alpha=16, sigma=0.02, layers=80, chain_silu=True),
}


@dataclass
class LinearInputs:
    W: torch.Tensor
    X: torch.Tensor
    A: torch.Tensor
    B: torch.Tensor
    dY: torch.Tensor
    scale: float
    meta: dict = field(default_factory=dict)


def linear_inputs(cid: int, layer: int, li: int, n: int, k: int, m: int, r: int, scale: float,
                  sigma: float = 0.02, outlier_frac: float = 0.0) -> LinearInputs:
    """All host tensors of one linear; seed tuple (config, layer*16 + linear, tensor)."""
    lid = layer * 16 + li
    W = weight_bf16(n, k, sigma, cid, lid, T_W, outlier_frac=outlier_frac)
    X = normal_bf16((m, k), 1.0, cid, lid, T_X)
    A = lora_A(r, k, cid, lid, T_A) if r > 0 else torch.zeros((0, k), dtype=torch.bfloat16)
    B = lora_B(n, r, cid, lid, T_B) if r > 0 else torch.zeros((n, 0), dtype=torch.bfloat16)
    dY = normal_bf16((m, n), 1.0, cid, lid, T_DY)
    return LinearInputs(W, X, A, B, dY, scale,
                        dict(config=cid, layer=layer, linear=li, n=n, k=k, m=m, r=r))


def device_linear_inputs(cid: int, layer: int, li: int, n: int, k: int, r: int, scale: float,
                         sigma: float = 0.02) -> LinearInputs:
    """W, A, B of one linear drawn on the device (same distributions and seed
    tuples as linear_inputs, torch's generator); X and dY are left to the
    caller (None)."""
    lid = layer * 16 + li
    W = device_normal_bf16((n, k), sigma, cid, lid, T_W)
    A = device_uniform_bf16((r, k), 1.0 / math.sqrt(k), cid, lid, T_A)
    B = device_normal_bf16((n, r), 0.01, cid, lid, T_B)
    return LinearInputs(W, None, A, B, None, scale, dict(config=cid, layer=layer, linear=li, n=n, k=k, m=None, r=r))


def config_linear_inputs(cid: int, li: int = 0, m: int | None = None, layer: int = 0) -> LinearInputs:
    c = CONFIGS[cid]
    lin = c.linears[li]
    return linear_inputs(cid, layer, li, lin.n, lin.k, c.m[0] if m is None else m, c.r, c.scale,
                         sigma=c.sigma, outlier_frac=c.outlier_frac)

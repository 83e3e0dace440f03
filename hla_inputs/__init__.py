"""Seeded synthetic inputs for masked second-order HLA.

This module is shared by the tests, the smoke check and the bench; it holds
none of the method's arithmetic (no moments, no scans, no outputs), only the
random tensors and the workload parameters, so the HIP path and the CPU
oracle always consume bit-identical inputs.

Recipe (the workloads are synthetic; no dataset is involved):
  * a CPU ``torch.Generator`` seeded with the given seed, draws in the order
    q, k, v (then, for a decode step, the new token's q, k, v);
  * each draw is ``torch.randn(shape, dtype=float32) * (1/sqrt(d))`` in fp32
    (1/sqrt(d) is applied to v too, with d the key width);
  * then rounded to bf16 (round-to-nearest-even) unless the workload is fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass
class Workload:
    name: str
    B: int
    H: int
    n: int
    d: int
    dv: int
    dtype: torch.dtype
    chunk: int = 0                     # 0 = library default
    gamma: Optional[List[float]] = None  # per head, exact fp32 values, or None
    ridge: float = 0.0
    normalize: bool = False
    extra: dict = field(default_factory=dict)


def gamma_list_fp32(values) -> List[float]:
    """Round decays to fp32 once; both sides then use exactly these values."""
    return [float(torch.tensor(x, dtype=torch.float32).item()) for x in values]


def ridge_fp32(x: float) -> float:
    return float(torch.tensor(x, dtype=torch.float32).item())


# The five workloads, by what they are.
SMALL_FP32 = Workload("masked_hla_fwd_B1_H1_n256_d16_fp32", 1, 1, 256, 16, 16, torch.float32)
FWD_D64 = Workload("masked_hla_fwd_B4_H8_n2048_d64_bf16_w64", 4, 8, 2048, 64, 64,
                   torch.bfloat16, chunk=64)
RATIO_DECAY_D64 = Workload(
    "masked_hla_ratio_decay_ridge_B8_H8_n4096_d64_bf16_w64", 8, 8, 4096, 64, 64,
    torch.bfloat16, chunk=64,
    gamma=gamma_list_fp32([1.0 - 2.0 ** -(5 + h) for h in range(8)]),
    ridge=ridge_fp32(1e-3), normalize=True)
LONG_D128 = Workload("masked_hla_fwd_decay_B1_H16_n65536_d128_bf16_w128", 1, 16, 65536,
                     128, 128, torch.bfloat16, chunk=128,
                     gamma=gamma_list_fp32([0.999] * 16))
DECODE_D128 = Workload("masked_hla_decode_4096_states_d128_prefix512", 256, 16, 512, 128, 128,
                       torch.bfloat16)

WORKLOADS = [SMALL_FP32, FWD_D64, RATIO_DECAY_D64, LONG_D128, DECODE_D128]


def draw(gen: torch.Generator, shape, d: int, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32) * (1.0 / math.sqrt(d))
    return x.to(dtype) if dtype != torch.float32 else x


def qkv(B: int, H: int, n: int, d: int, dv: int, dtype: torch.dtype, seed: int):
    """q, k [B,H,n,d] and v [B,H,n,dv] on the CPU, in ``dtype``."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    q = draw(gen, (B, H, n, d), d, dtype)
    k = draw(gen, (B, H, n, d), d, dtype)
    v = draw(gen, (B, H, n, dv), d, dtype)
    return q, k, v


def workload_qkv(w: Workload, seed: int):
    return qkv(w.B, w.H, w.n, w.d, w.dv, w.dtype, seed)


def qkv_on_device(B: int, H: int, n: int, d: int, dv: int, dtype: torch.dtype, seed: int,
                  device) -> tuple:
    """Same distribution as ``qkv`` but drawn by a seeded generator on
    ``device`` (for timing runs whose inputs are too large to draw on the
    host quickly; values differ from ``qkv``'s)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    s = 1.0 / math.sqrt(d)
    out = []
    for shape in ((B, H, n, d), (B, H, n, d), (B, H, n, dv)):
        x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device) * s
        out.append(x.to(dtype) if dtype != torch.float32 else x)
    return tuple(out)


def upstream(B: int, H: int, n: int, dv: int, seed: int) -> torch.Tensor:
    """A seeded upstream gradient dout [B,H,n,dv] in fp32 (standard normal draws
    from a CPU generator; the gradient of the loss with respect to out)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return torch.randn(B, H, n, dv, generator=gen, dtype=torch.float32)


def decode_inputs(B: int, H: int, prefix: int, d: int, dv: int, dtype: torch.dtype, seed: int):
    """Prefix q/k/v [B,H,prefix,·] then the new token's q/k/v [B,H,·]."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    q = draw(gen, (B, H, prefix, d), d, dtype)
    k = draw(gen, (B, H, prefix, d), d, dtype)
    v = draw(gen, (B, H, prefix, dv), d, dtype)
    q1 = draw(gen, (B, H, d), d, dtype)
    k1 = draw(gen, (B, H, d), d, dtype)
    v1 = draw(gen, (B, H, dv), d, dtype)
    return (q, k, v), (q1, k1, v1)


def random_state_fp32(N: int, d: int, dv: int, seed: int, scale: float = 1.0):
    """Arbitrary (not method-produced) fp32 summaries for compose tests:
    symmetric S, general C, m, G, h, and rho in (0.5, 1]."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    a = torch.randn(N, d, d, generator=gen) * scale
    S = (a + a.transpose(1, 2)) * 0.5
    C = torch.randn(N, d, dv, generator=gen) * scale
    m = torch.randn(N, d, generator=gen) * scale
    G = torch.randn(N, d, dv, generator=gen) * scale
    h = torch.randn(N, d, generator=gen) * scale
    rho = 0.5 + 0.5 * torch.rand(N, generator=gen)
    return S, C, m, G, h, rho

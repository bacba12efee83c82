"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it performs none of
the method's arithmetic.  Every tensor is created on the CPU from a seeded
``torch.Generator`` so that the oracle and the GPU library consume identical
bits (bf16 data is rounded once, here, by ``Tensor.to(torch.bfloat16)``).

Recipe (one seed per workload):
  * projected inputs x = [q | k | v] per token, each head-major:
    q, v ~ N(0, 1); raw k ~ N(0, 1) then L2-normalised per head; rounded to bf16;
  * conv taps ~ N(0, 0.5^2) per channel and tap (post-conv variance near 1), bf16;
  * alpha = sigmoid(N(3, 1)) per (token, head) or per (token, head, channel), fp32;
  * beta = sigmoid(N(0, 1)) per (token, head), fp32;
  * warm pool contents: ssm ~ N(0, 0.25^2), conv rows ~ N(0, 1), bf16 or fp32;
  * slot tables: distinct draws from [1, slots) (slot 0 is reserved).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

ALPHA_PER_HEAD, ALPHA_PER_CHANNEL = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    heads: int
    head_k: int
    head_v: int
    slots: int
    ssm_bf16: bool
    alpha_mode: int
    seed: int

    @property
    def channels(self) -> int:
        return self.heads * (2 * self.head_k + self.head_v)


# The five workloads, in the order the benchmark and the tests refer to them.
TINY = Workload("tiny fp32 check: H=2 K=V=16, 2x256 tokens", 1, 2, 16, 16, 8, False,
                ALPHA_PER_CHANNEL, 101)
GDN_DECODE = Workload("GDN decode: H=32 K=V=128, fp32 pool 512, batch 128", 1, 32, 128, 128,
                      512, False, ALPHA_PER_HEAD, 102)
KDA_PREFILL = Workload("KDA chunked prefill: H=12 K=V=128, 1x6144 tokens, bf16 pool", 1, 12,
                       128, 128, 8, True, ALPHA_PER_CHANNEL, 103)
KDA_DECODE = Workload("KDA decode with tracking: H=12 K=V=128, 69 layers, batch 256, bf16 pool",
                      69, 12, 128, 128, 1024, True, ALPHA_PER_CHANNEL, 104)
WARM_PREFILL = Workload("prefix-hit restore + warm prefill: H=32 K=V=128, 24 layers, fp32 pool",
                        24, 32, 128, 128, 81, False, ALPHA_PER_HEAD, 105)


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def projected_inputs(g: torch.Generator, tokens: int, heads: int, head_k: int, head_v: int,
                     alpha_mode: int) -> dict:
    """x bf16 [T, C]; alpha fp32 [T, H] or [T, H, K]; beta fp32 [T, H]."""
    q = torch.randn(tokens, heads, head_k, generator=g)
    k = torch.randn(tokens, heads, head_k, generator=g)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    v = torch.randn(tokens, heads, head_v, generator=g)
    x = torch.cat([q.reshape(tokens, -1), k.reshape(tokens, -1), v.reshape(tokens, -1)], dim=1)
    x = x.to(torch.bfloat16).contiguous()
    shape = (tokens, heads, head_k) if alpha_mode == ALPHA_PER_CHANNEL else (tokens, heads)
    alpha = torch.sigmoid(torch.randn(shape, generator=g) + 3.0).contiguous()
    beta = torch.sigmoid(torch.randn(tokens, heads, generator=g)).contiguous()
    return {"x": x, "alpha": alpha, "beta": beta}


def conv_weights(g: torch.Generator, channels: int) -> torch.Tensor:
    """bf16 [C, 4]; tap 3 multiplies the current token."""
    return (0.5 * torch.randn(channels, 4, generator=g)).to(torch.bfloat16).contiguous()


def distinct_slots(g: torch.Generator, n: int, slots: int) -> torch.Tensor:
    """n distinct slot ids drawn from [1, slots)."""
    if n > slots - 1:
        raise ValueError("not enough slots")
    return (torch.randperm(slots - 1, generator=g)[:n] + 1).to(torch.int32)


def warm_pool(g: torch.Generator, layers: int, slots: int, heads: int, head_k: int,
              head_v: int, ssm_bf16: bool):
    """Random pool contents: (ssm [L,N,H,V,K] fp32|bf16, conv [L,N,3,C] bf16)."""
    C = heads * (2 * head_k + head_v)
    ssm = 0.25 * torch.randn(layers, slots, heads, head_v, head_k, generator=g)
    ssm = ssm.to(torch.bfloat16 if ssm_bf16 else torch.float32).contiguous()
    conv = torch.randn(layers, slots, 3, C, generator=g).to(torch.bfloat16).contiguous()
    return ssm, conv


def cu_seqlens(lengths) -> torch.Tensor:
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 tensor (for the oracle)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")

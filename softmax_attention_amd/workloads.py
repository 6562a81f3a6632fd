"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and arranges them into the tensor
layouts the calls take; it holds none of the attention arithmetic.  Both the
HIP path (through the benchmark and the tests) and the CPU oracle (through the
tests) receive the very tensors built here, on the host, from a seeded
``torch.Generator('cpu')``.

Recipe for every named workload (the seed is the workload number):
  1. integers first: lengths, padding lengths, page permutations;
  2. then q, k, v in that order, each ``randn(shape) * sigma`` in float32,
     rounded to the 16-bit dtype with round-to-nearest-even (``.to(dtype)``).

The head geometries are shapes only: 32/8 query/KV heads with D = 128 is the
Qwen3-8B attention shape named on the RL-Kernel "Standard Softmax Attention"
page (Tensor Contract), and 24/2 heads with D = 256 is the canonical geometry
on the MATE "QSA" page (Core Attention).  No dataset or trained weight is
involved.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass
class Workload:
    name: str
    paged: bool
    dtype: torch.dtype
    B: int
    Sq: int
    Hq: int
    Hkv: int
    D: int
    causal: bool
    scale: Optional[float]
    q: torch.Tensor
    # dense
    Skv: int = 0
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    key_padding_mask: Optional[torch.Tensor] = None
    # paged
    k_cache: Optional[torch.Tensor] = None
    v_cache: Optional[torch.Tensor] = None
    real_seqlen_kv: Optional[torch.Tensor] = None
    block_table: Optional[torch.Tensor] = None
    page_size: int = 0

    def kv_lengths(self) -> list:
        if self.paged:
            return [int(x) for x in self.real_seqlen_kv.tolist()]
        return [self.Skv] * self.B


def _randn(g: torch.Generator, shape, sigma: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(dtype)


def dense_inputs(B, Sq, Skv, Hq, Hkv, D, *, dtype=torch.bfloat16, seed=0, sigma=1.0):
    """q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] drawn i.i.d. N(0, sigma^2) in that order."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = _randn(g, (B, Sq, Hq, D), sigma, dtype)
    k = _randn(g, (B, Skv, Hkv, D), sigma, dtype)
    v = _randn(g, (B, Skv, Hkv, D), sigma, dtype)
    return q, k, v


def scatter_to_pages(kd: torch.Tensor, block_table: torch.Tensor, page_size: int,
                     num_pages: int, fill: float = 0.0) -> torch.Tensor:
    """Place dense rows kd [B, S, Hkv, D] into a physical cache
    [num_pages * page_size, Hkv, D]: logical page p of request b goes to
    physical page block_table[b, p].  Rows no logical page maps to hold
    ``fill`` (tests fill them with sentinels that must never be read)."""
    B, S, Hkv, D = kd.shape
    cache = torch.full((num_pages * page_size, Hkv, D), fill, dtype=kd.dtype)
    n_logical = (S + page_size - 1) // page_size
    for b in range(B):
        for p in range(n_logical):
            lo, hi = p * page_size, min(S, (p + 1) * page_size)
            phys = int(block_table[b, p])
            cache[phys * page_size: phys * page_size + (hi - lo)] = kd[b, lo:hi]
    return cache


# --------------------------------------------------------------------------
# The five named workloads.


def tiny_dense_gqa() -> Workload:
    """Dense causal GQA, B=1, Hq=4, Hkv=2, Sq=Skv=64, D=64, bf16, scale 1/8."""
    q, k, v = dense_inputs(1, 64, 64, 4, 2, 64, dtype=torch.bfloat16, seed=1)
    return Workload("tiny_dense_gqa_b1_h4kv2_s64_d64", False, torch.bfloat16, 1, 64, 4, 2, 64,
                    True, 1.0 / 8.0, q, Skv=64, k=k, v=v)


def qwen3_8b_prefill() -> Workload:
    """Dense causal GQA prefill at the Qwen3-8B attention shape: B=2, Hq=32,
    Hkv=8, Sq=Skv=4096, D=128, bf16, scale 1/sqrt(128)."""
    q, k, v = dense_inputs(2, 4096, 4096, 32, 8, 128, dtype=torch.bfloat16, seed=2)
    return Workload("causal_gqa_prefill_b2_h32kv8_s4096_d128", False, torch.bfloat16, 2, 4096,
                    32, 8, 128, True, 1.0 / math.sqrt(128.0), q, Skv=4096, k=k, v=v)


def paged_decode() -> Workload:
    """Paged decode: B=64, Sq=1, Hq=32, Hkv=8, D=128, page 64, bf16; lengths
    uniform in [512, 8192]; block_table [64, 128] from a permutation of the
    8192 physical pages; K/V caches [8192*64, 8, 128] drawn directly."""
    g = torch.Generator("cpu").manual_seed(3)
    lens = torch.randint(512, 8193, (64,), generator=g, dtype=torch.int64).to(torch.int32)
    bt = torch.randperm(8192, generator=g).view(64, 128).to(torch.int32)
    q = _randn(g, (64, 1, 32, 128), 1.0, torch.bfloat16)
    kc = _randn(g, (8192 * 64, 8, 128), 1.0, torch.bfloat16)
    vc = _randn(g, (8192 * 64, 8, 128), 1.0, torch.bfloat16)
    return Workload("paged_decode_b64_h32kv8_d128_page64", True, torch.bfloat16, 64, 1, 32, 8,
                    128, True, None, q, k_cache=kc, v_cache=vc, real_seqlen_kv=lens,
                    block_table=bt, page_size=64)


def mha_key_padding() -> Workload:
    """Non-causal MHA with key padding: B=4, H=16, S=2048, D=64, fp16, sigma
    0.5; key_padding_mask keeps the first L_b keys, L_b uniform in
    [1024, 2048]; scale 1/8."""
    g = torch.Generator("cpu").manual_seed(4)
    L = torch.randint(1024, 2049, (4,), generator=g)
    q = _randn(g, (4, 2048, 16, 64), 0.5, torch.float16)
    k = _randn(g, (4, 2048, 16, 64), 0.5, torch.float16)
    v = _randn(g, (4, 2048, 16, 64), 0.5, torch.float16)
    mask = torch.arange(2048)[None, :] < L[:, None]
    return Workload("mha_key_padding_b4_h16_s2048_d64", False, torch.float16, 4, 2048, 16, 16,
                    64, False, 1.0 / 8.0, q, Skv=2048, k=k, v=v, key_padding_mask=mask)


def wide_group_chunked_prefill() -> Workload:
    """Chunked prefill through the paged path: B=2, Hq=24, Hkv=2 (group 12),
    D=256, Sq=512 new queries at the end of 16384 cached keys, bf16, scale
    1/16, page 64, block_table from a permutation of the 512 physical pages."""
    g = torch.Generator("cpu").manual_seed(5)
    bt = torch.randperm(512, generator=g).view(2, 256).to(torch.int32)
    q = _randn(g, (2, 512, 24, 256), 1.0, torch.bfloat16)
    kd = _randn(g, (2, 16384, 2, 256), 1.0, torch.bfloat16)
    vd = _randn(g, (2, 16384, 2, 256), 1.0, torch.bfloat16)
    kc = scatter_to_pages(kd, bt, 64, 512)
    vc = scatter_to_pages(vd, bt, 64, 512)
    lens = torch.tensor([16384, 16384], dtype=torch.int32)
    return Workload("wide_group_chunked_prefill_b2_h24kv2_d256_q512_kv16384", True,
                    torch.bfloat16, 2, 512, 24, 2, 256, True, 1.0 / 16.0, q, k_cache=kc,
                    v_cache=vc, real_seqlen_kv=lens, block_table=bt, page_size=64)


WORKLOADS = {
    1: tiny_dense_gqa,
    2: qwen3_8b_prefill,
    3: paged_decode,
    4: mha_key_padding,
    5: wide_group_chunked_prefill,
}


def make(n: int) -> Workload:
    return WORKLOADS[n]()

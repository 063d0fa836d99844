"""Seeded synthetic inputs for the tests, ``smoke()`` and ``bench.py``.

This module draws random numbers and states workload sizes; it holds none of
the method's arithmetic (no attention, no translation, no block management)
and imports neither the oracle nor the product library.  Both sides of every
parity test consume exactly what it returns.

Workloads (shapes and distributions of the pages' 8B-style GQA example:
32 layers, 8 KV heads, d_head 128, 2-byte elements):
  tiny     4 sequences of {17, 33, 64, 100} tokens, Hq 8, Hkv 2, d 64, B 16,
           64-block pool, fp32, q/K/V ~ N(0, 1)
  gqa8b    64 sequences, lengths uniform in [512, 4096], Hq 32, Hkv 8, d 128,
           B 16, pool = 1.25 x the blocks the lengths need, bf16,
           q/K/V ~ N(0, 1) / sqrt(d)
  sweep    256 sequences of 4096 - r tokens, r uniform in [0, B), B in
           {8, 16, 32}, pool x 1.25, bf16, N(0, 1) / sqrt(d)
  fork     32 prompts of 2055 tokens, each forked into 8 samples, 16 steps of
           append + decode, bf16, N(0, 1) / sqrt(d)
  long     32 layers, 16 sequences of 32768 tokens, B 16, 32768-block pool
           (64 GiB of K and V), bf16, N(0, 1) / sqrt(d)
Values are drawn in fp32 and rounded once to the storage type; both sides
read those stored values.

FP8 caches (E4M3 codes with per-(block, KV head) scales) are drawn as codes
directly: random sign, exponent field round(N(12, 1)) clamped to [0, 15],
uniform mantissa, the NaN magnitude 0x7F replaced by 0x7E -- the shape of
amax-scaled normal data -- and fp32 scales value_scale / 78 * U(0.5, 2) per
(block, KV head), 78 being the RMS of those code values, so that the values
the cache stands for have an RMS of about value_scale.

INT8 caches (signed codes with per-(block, KV head) scales) are drawn as codes
round(N(0, 36^2)) clamped to -127..127 -- amax-scaled normal data, the largest
of a block's 2048 values (about 3.5 standard deviations) near 127 -- and fp32
scales value_scale / 36 * U(0.5, 2), for values of RMS about value_scale.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    hq: int
    hkv: int
    d: int
    block_size: int
    dtype: str            # "f32" or "bf16"
    seed: int
    layers: int = 1
    pool_factor: float = 1.25
    value_scale: float = 1.0
    fixed_lens: Optional[List[int]] = field(default=None)
    fixed_pool_blocks: Optional[int] = None

    @property
    def scale(self) -> float:  # the textbook 1 / sqrt(d_head)
        return 1.0 / math.sqrt(self.d)


def tiny() -> Workload:
    return Workload("tiny", 4, 8, 2, 64, 16, "f32", 1001, fixed_lens=[17, 33, 64, 100],
                    fixed_pool_blocks=64)


def gqa8b() -> Workload:
    return Workload("gqa8b", 64, 32, 8, 128, 16, "bf16", 1002, value_scale=1.0 / math.sqrt(128))


def sweep(block_size: int) -> Workload:
    return Workload(f"sweep_b{block_size}", 256, 32, 8, 128, block_size, "bf16", 1003 + block_size,
                    value_scale=1.0 / math.sqrt(128))


def fork() -> Workload:
    return Workload("fork", 256, 32, 8, 128, 16, "bf16", 1004, value_scale=1.0 / math.sqrt(128),
                    fixed_lens=[2055] * 32)


def long() -> Workload:
    return Workload("long", 16, 32, 8, 128, 16, "bf16", 1005, layers=32, value_scale=1.0 / math.sqrt(128),
                    fixed_lens=[32768] * 16, fixed_pool_blocks=32768)


FORK_PROMPTS = 32
FORK_SAMPLES = 8
FORK_STEPS = 16


def seq_lengths(w: Workload) -> List[int]:
    """Context length of every sequence (seeded)."""
    if w.fixed_lens is not None:
        return list(w.fixed_lens)
    rng = np.random.default_rng(w.seed)
    if w.name == "gqa8b":
        return [int(x) for x in rng.integers(512, 4096, size=w.num_seqs, endpoint=True)]
    if w.name.startswith("sweep"):
        return [4096 - int(x) for x in rng.integers(0, w.block_size, size=w.num_seqs)]
    raise ValueError(w.name)


def pool_blocks(w: Workload, lens: List[int], extra: int = 0) -> int:
    """Pool size: fixed, or pool_factor x the blocks the lengths occupy (plus extra)."""
    if w.fixed_pool_blocks is not None:
        return w.fixed_pool_blocks + extra
    occupied = sum((s + w.block_size - 1) // w.block_size for s in lens) + extra
    return int(math.ceil(w.pool_factor * occupied))


def pop_order(num_blocks: int, seed: int) -> np.ndarray:
    """Seeded random permutation of the block ids: the order in which free blocks are first handed out."""
    return np.random.default_rng(seed + 7919).permutation(num_blocks).astype(np.int32)


def torch_dtype(w: Workload):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def randn(shape, dtype, scale: float, seed: int, device="cpu"):
    """N(0, 1) * scale drawn in fp32 with a seeded generator, rounded once to `dtype`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def fill_randn_(t, scale: float, seed: int, chunk_rows: int = 0):
    """Fill an existing tensor in place, chunk by chunk along dim 0 (seed per chunk), N(0,1)*scale.

    Keeps the fp32 temporary small for very large pools.
    """
    import torch
    rows = t.shape[0]
    if chunk_rows <= 0:
        per_row = max(1, t[0].numel())
        chunk_rows = max(1, (1 << 28) // (per_row * 4))  # ~1 GiB of fp32 per chunk
    g = torch.Generator(device=t.device)
    for i, start in enumerate(range(0, rows, chunk_rows)):
        stop = min(rows, start + chunk_rows)
        g.manual_seed(seed * 1000003 + i)
        x = torch.randn(t[start:stop].shape, generator=g, dtype=torch.float32, device=t.device)
        if scale != 1.0:
            x.mul_(scale)
        t[start:stop].copy_(x)
        del x
    return t


FP8_CODE_RMS = 78.0


def fill_fp8_codes_(t, seed: int, chunk_rows: int = 0):
    """Fill a uint8 tensor in place with random E4M3 codes (no NaN codes); see the module docstring.

    Drawn on the tensor's device, chunk by chunk along dim 0 (seed per chunk).
    """
    import torch
    rows = t.shape[0]
    if chunk_rows <= 0:
        chunk_rows = max(1, (1 << 26) // max(1, t[0].numel()))
    g = torch.Generator(device=t.device)
    for i, start in enumerate(range(0, rows, chunk_rows)):
        stop = min(rows, start + chunk_rows)
        g.manual_seed(seed * 1000003 + i)
        shape = tuple(t[start:stop].shape)
        sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32, device=t.device)
        expo = torch.round(torch.randn(shape, generator=g, device=t.device) + 12.0).clamp_(0, 15).to(torch.int32)
        mant = torch.randint(0, 8, shape, generator=g, dtype=torch.int32, device=t.device)
        mag = expo * 8 + mant
        mag = torch.where(mag == 0x7F, torch.full_like(mag, 0x7E), mag)
        t[start:stop].copy_((sign * 0x80 + mag).to(torch.uint8))
    return t


INT8_CODE_RMS = 36.0


def fill_int8_codes_(t, seed: int, chunk_rows: int = 0):
    """Fill a uint8 tensor in place with random INT8 codes (two's complement bytes); see the module docstring.

    Drawn on the tensor's device, chunk by chunk along dim 0 (seed per chunk).
    """
    import torch
    rows = t.shape[0]
    if chunk_rows <= 0:
        chunk_rows = max(1, (1 << 26) // max(1, t[0].numel()))
    g = torch.Generator(device=t.device)
    for i, start in enumerate(range(0, rows, chunk_rows)):
        stop = min(rows, start + chunk_rows)
        g.manual_seed(seed * 1000003 + i)
        shape = tuple(t[start:stop].shape)
        c = torch.round(torch.randn(shape, generator=g, device=t.device) * INT8_CODE_RMS).clamp_(-127, 127)
        t[start:stop].copy_(c.to(torch.int32).bitwise_and(0xFF).to(torch.uint8))
    return t


def int8_scales(num_blocks: int, hkv: int, value_scale: float, seed: int, device="cpu"):
    """float32 [num_blocks][hkv] scales value_scale / INT8_CODE_RMS * U(0.5, 2)."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    u = torch.rand((num_blocks, hkv), generator=g) * 1.5 + 0.5
    return (u * (value_scale / INT8_CODE_RMS)).to(torch.float32).to(device)


def fp8_scales(num_blocks: int, hkv: int, value_scale: float, seed: int, device="cpu"):
    """float32 [num_blocks][hkv] scales value_scale / FP8_CODE_RMS * U(0.5, 2)."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    u = torch.rand((num_blocks, hkv), generator=g) * 1.5 + 0.5
    return (u * (value_scale / FP8_CODE_RMS)).to(torch.float32).to(device)

"""KV sizing, block-table footprint, tail waste and capacity arithmetic.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain integer
arithmetic written from the pages; the tests pin each function to the numbers
the pages print.
"""

from __future__ import annotations

from fractions import Fraction
from typing import Dict, Sequence


def kv_bytes_per_token(layers: int, kv_heads: int, d_head: int, elem_bytes: int) -> int:
    """2 (keys and values) * L * H_kv * d_head * sizeof(dtype) -- [P1] section 1."""
    return 2 * layers * kv_heads * d_head * elem_bytes


def sequence_kv_bytes(tokens: int, layers: int, kv_heads: int, d_head: int, elem_bytes: int) -> int:
    """KV bytes of one sequence: tokens * bytes per token -- [P1] section 1, [P2] section 4."""
    return tokens * kv_bytes_per_token(layers, kv_heads, d_head, elem_bytes)


def blocks_needed(tokens: int, block_size: int) -> int:
    """ceil(S / B) blocks for S cached tokens -- [P1] section 8 item 3."""
    return -(-tokens // block_size)


def tail_waste(tokens: int, block_size: int) -> int:
    """Unused slots of the last block: ceil(S/B)*B - S -- [P1] section 8 item 3."""
    return blocks_needed(tokens, block_size) * block_size - tokens


def block_table_bytes(tokens: int, block_size: int, entry_bytes: int = 4) -> int:
    """Size of one sequence's block table (int32 entries) -- [P1] section 8 'Block table metadata footprint'."""
    return blocks_needed(tokens, block_size) * entry_bytes


def table_to_payload_ratio(tokens: int, block_size: int, bytes_per_token: int) -> Fraction:
    """Block-table bytes over the KV bytes they map, as an exact fraction."""
    return Fraction(block_table_bytes(tokens, block_size), tokens * bytes_per_token)


def capacity_plan(lengths: Sequence[int], block_size: int, pool_bytes: int,
                  bytes_per_slot: int) -> Dict[str, object]:
    """Does a batch of sequence lengths fit a pool?  [P1] sections 10 and 23.

    The pool holds pool_bytes // bytes_per_slot token slots; every sequence
    takes ceil(S/B) whole blocks.
    """
    pool_slots = pool_bytes // bytes_per_slot
    blocks = [blocks_needed(s, block_size) for s in lengths]
    slots = sum(b * block_size for b in blocks)
    waste = sum(tail_waste(s, block_size) for s in lengths)
    return {
        "pool_slots": pool_slots,
        "blocks": sum(blocks),
        "slots": slots,
        "waste": waste,
        "waste_fraction": Fraction(waste, slots) if slots else Fraction(0),
        "fits": slots <= pool_slots,
        "memory_bytes": slots * bytes_per_slot,
        "deficit_slots": max(0, slots - pool_slots),
    }


def kv_cache_gb(n_layers: int, n_heads: int, head_dim: int, seq_len: int, batch: int,
                bytes_per_elem: int = 2) -> float:
    """[P3]'s sizing helper: 2 * layers * heads * head_dim * bytes * seq_len * batch / 1e9.

    Note the page multiplies by the number of (key/value) heads it is given and
    reports decimal gigabytes.
    """
    per_token = 2 * n_layers * n_heads * head_dim * bytes_per_elem
    return per_token * seq_len * batch / 1e9

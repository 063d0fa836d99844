"""fp64 reference for a KV cache stored as 8-bit integer codes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.

What the pages fix and what is read into them
---------------------------------------------
[P3] "Alternatives and ecosystem" names INT8 beside FP8 as a quantized KV
format that cuts bytes per token and combines with the paged layout; [P2]
sections 8 and 11 keep exactness claims for paging at the cache's own
precision.  As for the FP8 cache, the attention of an INT8 cache is the exact
attention over the values the cache holds: the oracle dequantizes every
stored code and runs the ordinary fp64 paged decode of ``oracle.attention``.

The pages fix neither the integer range nor the scaling.  Readings taken
here:
  * Codes: signed 8-bit two's complement integers; a stored code c stands for
    c * scale.  The appender writes only -127 .. 127 (symmetric, so negating
    a value negates its code); a stored -128 still stands for -128 * scale.
  * Scaling: as for the FP8 cache, one positive fp32 scale per (physical
    block, KV head) for keys and another for values, owned by the caller.
  * Quantizing x with scale s: the integer nearest to the real number x / s,
    ties to the even integer, clamped to -127 .. 127.  An 8-bit integer has no
    NaN: NaN input, or a scale that is not positive and finite, stores 0.
  * Copy-on-write clones a block's codes together with its scales.

Layout: as in ``oracle.attention``, pools are logical
``[num_blocks][Hkv][block_size][d_head]`` (uint8 bytes holding the codes)
and scales are ``[num_blocks][Hkv]``.
"""

from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

from . import attention as OA

MAX_CODE = 127


def code_value(code: int) -> int:
    """The integer a stored byte stands for (two's complement): 0..127 as is, 128..255 as byte - 256."""
    code = int(code) & 0xFF
    return code - 256 if code >= 128 else code


def value_table() -> np.ndarray:
    """Values of all 256 bytes, float64."""
    return np.array([code_value(c) for c in range(256)], dtype=np.float64)


_TABLE = value_table()


def quantize_one(x: float, s: float) -> int:
    """Byte holding the code of x under scale s.

    The quotient x / s is formed in fp64.  x and s hold at most 24 significant
    bits each, so the exact quotient is either itself a half-integer (then the
    fp64 quotient is exact) or at least about 2^-33 (relative) away from every
    half-integer, far more than the fp64 rounding of the quotient (2^-53): the
    nearest-integer decision below is the one the exact quotient gives.
    """
    x = float(x)
    s = float(s)
    if not (s > 0.0 and math.isfinite(s)) or math.isnan(x):
        return 0
    y = x / s
    if y >= MAX_CODE:  # includes +inf
        return MAX_CODE
    if y <= -MAX_CODE:
        return (-MAX_CODE) & 0xFF
    lo = math.floor(y)
    d_lo, d_hi = y - lo, (lo + 1) - y
    if d_lo < d_hi:
        q = lo
    elif d_hi < d_lo:
        q = lo + 1
    else:  # exact tie: the even neighbour
        q = lo if lo % 2 == 0 else lo + 1
    return int(q) & 0xFF


def quantize(x: np.ndarray, s: float) -> np.ndarray:
    """Elementwise ``quantize_one`` over an array, one scale; uint8 bytes."""
    flat = np.asarray(x, dtype=np.float64).ravel()
    return np.array([quantize_one(v, s) for v in flat], dtype=np.uint8).reshape(np.shape(x))


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Logical pool of bytes [nb][Hkv][B][d] and scales [nb][Hkv] -> fp64 values."""
    vals = _TABLE[np.asarray(codes, dtype=np.uint8)]
    return vals * np.asarray(scales, dtype=np.float64)[:, :, None, None]


def append_kv(k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray, v_scales: np.ndarray,
              k_new: np.ndarray, v_new: np.ndarray, slot_mapping: Sequence[int]) -> None:
    """Quantize token t's K/V (all KV heads) into slot ``slot_mapping[t]``, in place.

    The storage rule of ``oracle.attention.append_kv`` ([P1] section 16: the
    token goes to block slot // B at offset slot % B), each value encoded under
    the scale of its destination (block, KV head).  Negative slots and slots
    beyond the pool are skipped.
    """
    nb, hkv, block_size, _ = k_codes.shape
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0 or slot >= nb * block_size:
            continue
        pb, off = slot // block_size, slot % block_size
        for j in range(hkv):
            k_codes[pb, j, off, :] = quantize(k_new[t, j], k_scales[pb, j])
            v_codes[pb, j, off, :] = quantize(v_new[t, j], v_scales[pb, j])


def copy_blocks(k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray, v_scales: np.ndarray,
                pairs: Sequence[Tuple[int, int]]) -> None:
    """Copy-on-write clone ([P1] sections 15-16): codes and scales of block src over block dst."""
    OA.copy_blocks(k_codes, v_codes, pairs)
    for src, dst in pairs:
        k_scales[dst] = k_scales[src]
        v_scales[dst] = v_scales[src]


def paged_decode(q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray,
                 v_scales: np.ndarray, block_tables: np.ndarray, context_lens: Sequence[int],
                 scale: float) -> np.ndarray:
    """Decode attention over an INT8 cache: dequantize, then the fp64 paged decode."""
    return OA.paged_decode(q, dequantize(k_codes, k_scales), dequantize(v_codes, v_scales),
                           block_tables, context_lens, scale)

"""fp64 reference for a KV cache stored as 8-bit floating point codes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.

What the pages fix and what is read into them
---------------------------------------------
[P3] "Alternatives and ecosystem" names quantized KV (INT8/FP8) as the way to
cut bytes per token, to be combined with paged layout.  [P2] section 8 notes
that quantization changes precision, and that exactness claims for paging are
made at the same KV precision (section 11 of the same page says quantized
KV is a precision tradeoff of its own).  So the attention of a quantized cache is the exact attention over the
values the cache holds: the oracle dequantizes every stored code and then runs
the ordinary fp64 paged decode of ``oracle.attention``.

The pages do not name the 8-bit format or the scaling.  Readings taken
here:
  * Format: FP8 E4M3 as in the OCP 8-bit floating point specification -- one
    sign bit, four exponent bits with bias 7, three mantissa bits, subnormals
    at exponent field 0, no infinities, and the two codes 0x7F / 0xFF (all
    exponent and mantissa bits set) as NaN.  Largest finite magnitude 448.
  * Scaling: one positive fp32 scale per (physical block, KV head) for keys
    and another for values; a stored code c stands for value(c) * scale.
  * Quantizing x with scale s: the sign of x, and the finite magnitude code
    nearest to the real number |x| / s, ties to the code whose last mantissa
    bit is 0; magnitudes beyond 448 give 448 (saturation).  NaN inputs give
    the NaN code 0x7F.  A scale that is not positive and finite gives 0x7F.
  * Copy-on-write clones a block's codes together with its scales.

Layout: as in ``oracle.attention``, pools are logical
``[num_blocks][Hkv][block_size][d_head]`` (uint8 codes here) and scales are
``[num_blocks][Hkv]``.
"""

from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

from . import attention as OA

EXP_BIAS = 7
MAX_FINITE = 448.0
NAN_CODE = 0x7F
MAX_CODE = 0x7E  # 448


def code_value(code: int) -> float:
    """Real value of one E4M3 code (float('nan') for the NaN codes).

    sign * 2^(e - 7) * (1 + m / 8) for exponent field e >= 1, and
    sign * 2^(-6) * (m / 8) for e = 0 (subnormals and zeros).
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * math.ldexp(m / 8.0, 1 - EXP_BIAS)
    return sign * math.ldexp(1.0 + m / 8.0, e - EXP_BIAS)


def value_table() -> np.ndarray:
    """Values of all 256 codes, float64 (NaN at 0x7F and 0xFF)."""
    return np.array([code_value(c) for c in range(256)], dtype=np.float64)


_TABLE = value_table()
# finite non-negative magnitudes: codes 0x00 .. 0x7E, in increasing order of value
_MAGS = _TABLE[:NAN_CODE]


def quantize_one(x: float, s: float) -> int:
    """Code of x under scale s, by nearest-value search over the finite codes.

    The quotient |x| / s is formed in fp64.  x holds at most 24 significant
    bits and s 24, so when the exact quotient is not itself a midpoint between
    two neighbouring magnitudes it lies at least 2^-30 (relative) away from
    every midpoint, far more than the fp64 rounding of the quotient (2^-53):
    the nearest-code decision below is the one the exact quotient gives.
    """
    x = float(x)
    s = float(s)
    if not (s > 0.0 and math.isfinite(s)) or math.isnan(x):
        return NAN_CODE
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    y = abs(x) / s
    if y >= MAX_FINITE:  # includes +inf
        return sign | MAX_CODE
    # nearest magnitude; on an exact tie take the code with even mantissa
    dist = np.abs(_MAGS - y)
    best = int(np.argmin(dist))
    ties = np.flatnonzero(dist == dist[best])
    if len(ties) > 1:
        best = int(next(c for c in ties if (c & 1) == 0))
    return sign | best


def quantize(x: np.ndarray, s: float) -> np.ndarray:
    """Elementwise ``quantize_one`` over an array, one scale; uint8 codes."""
    flat = np.asarray(x, dtype=np.float64).ravel()
    return np.array([quantize_one(v, s) for v in flat], dtype=np.uint8).reshape(np.shape(x))


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Logical pool of codes [nb][Hkv][B][d] and scales [nb][Hkv] -> fp64 values."""
    vals = _TABLE[np.asarray(codes, dtype=np.uint8)]
    return vals * np.asarray(scales, dtype=np.float64)[:, :, None, None]


def append_kv(k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray, v_scales: np.ndarray,
              k_new: np.ndarray, v_new: np.ndarray, slot_mapping: Sequence[int]) -> None:
    """Quantize token t's K/V (all KV heads) into slot ``slot_mapping[t]``, in place.

    The storage rule of ``oracle.attention.append_kv`` ([P1] section 16: the
    token goes to block slot // B at offset slot % B), with each value encoded
    under the scale of its destination (block, KV head).  Negative slots and
    slots beyond the pool are skipped.
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
    """Decode attention over a quantized cache: dequantize, then the fp64 paged decode."""
    return OA.paged_decode(q, dequantize(k_codes, k_scales), dequantize(v_codes, v_scales),
                           block_tables, context_lens, scale)

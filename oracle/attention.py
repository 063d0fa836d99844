"""fp64 reference for paged decode attention and its storage rules.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.  Everything here is NumPy in float64 on the CPU and works on the
logical pool layout

    k_pool, v_pool : [num_blocks][num_kv_heads][block_size][d_head]

so that ``k_pool[pb, j, off, :]`` is the key of the token stored in slot
``off`` of physical block ``pb`` for KV head ``j``.

Readings of the pages taken here:
  * GQA head mapping: query head ``h`` reads KV head ``h // (Hq // Hkv)``
    (consecutive query heads share a KV head).  [P2] section 7 only says that
    several query heads share one KV head.
  * ``scale`` is supplied by the caller; the attention formula of [P1]
    section 1 and [P2] section 10 uses 1/sqrt(d_head).
  * A sequence of length 0 attends to nothing; its output is defined as zeros.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# Address translation -- [P1] section 7 "Address translation arithmetic";
# [P2] section 5 (token t -> logical block floor(t/B), slot t mod B).
# ---------------------------------------------------------------------------

def translate(i: int, block_size: int, block_table: Sequence[int]) -> Tuple[int, int, int, int]:
    """Map zero-based token index ``i`` to (logical block, offset, physical block, slot).

    logical block = floor(i / block_size), offset = i mod block_size,
    physical block = block_table[logical block]  ([P1] section 7);
    slot = physical block * block_size + offset, i.e. the position of the token
    in the flat slot space of the pool ([P2] section 2: the frame times the page
    size plus the unchanged offset).
    """
    if i < 0 or block_size <= 0:
        raise ValueError("token index must be >= 0 and block_size > 0")
    lb = i // block_size
    off = i % block_size
    pb = int(block_table[lb])
    return lb, off, pb, pb * block_size + off


# ---------------------------------------------------------------------------
# Attention -- [P1] section 1 (softmax(q K^T / sqrt(d_head)) V for one query
# token over S cached positions); [P2] section 10 (s = q K^T / sqrt(d),
# a_i = exp(s_i) / sum_j exp(s_j), o = sum_i a_i v_i) and section 11 (the
# common-maximum shift that keeps exp finite).
# ---------------------------------------------------------------------------

def gather_sequence(pool: np.ndarray, block_table: Sequence[int], seq_len: int,
                    kv_head: int) -> np.ndarray:
    """Rows of one KV head for tokens 0..seq_len-1, in logical order.

    Walks the logical blocks b = 0 .. ceil(S/B)-1 ([P1] section 13 step 2) and
    takes only the valid slots of each: all B slots of a full block, S - b*B
    slots of the last one.  Tail slots past S are never read.
    """
    block_size = pool.shape[2]
    n_blocks = -(-seq_len // block_size)
    rows = []
    for b in range(n_blocks):
        pb = int(block_table[b])
        valid = block_size if b < n_blocks - 1 else seq_len - b * block_size
        rows.append(pool[pb, kv_head, :valid, :])
    if not rows:
        return np.zeros((0, pool.shape[3]), dtype=np.float64)
    return np.concatenate(rows, axis=0).astype(np.float64)


def softmax_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                      scale: float) -> np.ndarray:
    """One query vector against S key/value rows, fp64.

    s = scale * (keys @ q); m = max s; w = exp(s - m); o = (w @ values) / sum w.
    Subtracting the common maximum does not change the result ([P2] section 11).
    Returns zeros when S = 0 (nothing to attend to).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    s = scale * (keys @ q)
    m = np.max(s)
    w = np.exp(s - m)
    return (w @ values) / np.sum(w)


def attention_weights(q: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """The softmax weights a_i of [P2] section 10 (they sum to one)."""
    s = scale * (np.asarray(keys, dtype=np.float64) @ np.asarray(q, dtype=np.float64))
    w = np.exp(s - np.max(s))
    return w / np.sum(w)


def paged_decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                 block_tables: np.ndarray, context_lens: Sequence[int],
                 scale: float) -> np.ndarray:
    """Paged decode attention, fp64.

    q            [N][Hq][d]
    k_pool/v_pool [num_blocks][Hkv][B][d] (logical layout)
    block_tables [N][max_blocks] int
    context_lens [N]
    returns      [N][Hq][d] float64

    For every sequence n and query head h (KV head j = h // (Hq/Hkv)), gather
    K and V through the block table in logical order ([P1] sections 7 and 13)
    and evaluate softmax(scale * q K^T) V ([P1] section 1, [P2] section 10).
    """
    q = np.asarray(q, dtype=np.float64)
    n_seqs, hq, d = q.shape
    hkv = k_pool.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    out = np.zeros((n_seqs, hq, d), dtype=np.float64)
    for n in range(n_seqs):
        s_len = int(context_lens[n])
        for j in range(hkv):
            keys = gather_sequence(k_pool, block_tables[n], s_len, j)
            vals = gather_sequence(v_pool, block_tables[n], s_len, j)
            for h in range(j * group, (j + 1) * group):
                out[n, h] = softmax_attention(q[n, h], keys, vals, scale)
    return out


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Unpaged attention over contiguous K/V, written separately from the paged path.

    q [Hq][d]; k, v [S][Hkv][d] (contiguous, logical token order).  Evaluated
    head by head with explicit per-token loops for the scores, so that it does
    not reuse ``softmax_attention``; it is the "contiguous equivalent" that the
    pages compare the paged result against ([P1] section 20 test 3; [P2]
    section 10: the split calculation includes the same terms).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    s_len, hkv, _ = k.shape
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    if s_len == 0:
        return out
    for h in range(hq):
        j = h // group
        scores = np.array([scale * float(np.dot(q[h], k[t, j])) for t in range(s_len)])
        top = scores.max()
        e = np.exp(scores - top)
        out[h] = (e[:, None] * v[:, j, :]).sum(axis=0) / e.sum()
    return out


# ---------------------------------------------------------------------------
# Per-block summaries and their merge -- [P2] section 10 (unnormalised page
# sums N, Z) and section 11 (stable summaries m_b, z_b, u_b and the merge
# m = max m_b, z = sum exp(m_b - m) z_b, u = sum exp(m_b - m) u_b, o = u / z).
# ---------------------------------------------------------------------------

def page_sums(scores: np.ndarray, values: np.ndarray) -> Tuple[float, np.ndarray]:
    """Unshifted page sums of [P2] section 10: Z = sum exp(s_i), N = sum exp(s_i) v_i."""
    e = np.exp(np.asarray(scores, dtype=np.float64))
    return float(e.sum()), e @ np.asarray(values, dtype=np.float64)


def block_summary(scores: np.ndarray, values: np.ndarray) -> Tuple[float, float, np.ndarray]:
    """(m_b, z_b, u_b) of one block: its max score, shifted weight sum, shifted value sum."""
    s = np.asarray(scores, dtype=np.float64)
    m = float(np.max(s))
    e = np.exp(s - m)
    return m, float(e.sum()), e @ np.asarray(values, dtype=np.float64)


def merge_summaries(summaries: List[Tuple[float, float, np.ndarray]]) -> Tuple[float, float, np.ndarray]:
    """Merge block summaries into (m, z, u) with the common maximum of [P2] section 11."""
    m = max(s[0] for s in summaries)
    z = sum(math.exp(mb - m) * zb for mb, zb, _ in summaries)
    u = sum(math.exp(mb - m) * ub for mb, _, ub in summaries)
    return m, z, u


# ---------------------------------------------------------------------------
# Storage rules of the pool -- [P1] section 16 (a token's K/V is written into
# its block at its offset; copy-on-write clones the shared tail block) and
# section 20's teaching model (payload written at storage[block][offset]).
# ---------------------------------------------------------------------------

def append_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              slot_mapping: Sequence[int]) -> None:
    """Write token t's K/V (all KV heads) into slot ``slot_mapping[t]``, in place.

    slot = physical block * B + offset; negative slots are skipped.
    k_new, v_new: [T][Hkv][d].
    """
    block_size = k_pool.shape[2]
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        pb, off = slot // block_size, slot % block_size
        k_pool[pb, :, off, :] = k_new[t]
        v_pool[pb, :, off, :] = v_new[t]


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs: Sequence[Tuple[int, int]]) -> None:
    """Clone whole blocks for copy-on-write: pool[dst] = pool[src], in place.

    The page copies the valid tokens of the shared tail ([P1] sections 15-16);
    copying the whole block is a superset of that and leaves the valid slots
    identical.  Pools may carry a leading layer axis ``[L][num_blocks]...``.
    """
    layered = k_pool.ndim == 5
    for src, dst in pairs:
        if layered:
            k_pool[:, dst] = k_pool[:, src]
            v_pool[:, dst] = v_pool[:, src]
        else:
            k_pool[dst] = k_pool[src]
            v_pool[dst] = v_pool[src]

"""Pins for oracle/fp8.py: the E4M3 code values, the quantizer, the storage rules and the decode.

The code values and the round-to-nearest-even conversion are checked against
closed forms of the OCP E4M3 format and against PyTorch's own float8_e4m3fn
conversion (a library routine independent of the oracle); the quantizer's
fp64 decision against exact rational arithmetic; the decode against the
separately written dense attention over K/V dequantized token by token.
"""

import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F


def _torch_values(codes):
    return torch.as_tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


# ---- code values --------------------------------------------------------------

def test_code_values_closed_forms():
    v = F.value_table()
    assert v[0x7E] == 448.0                      # largest finite
    assert v[0x08] == 2.0 ** -6                  # smallest normal
    assert v[0x01] == 2.0 ** -9                  # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9              # largest subnormal
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x3F] == 1.875 and v[0x40] == 2.0
    assert v[0x00] == 0.0 and math.copysign(1.0, v[0x80]) < 0 and v[0x80] == 0.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and int(np.isnan(v).sum()) == 2
    assert np.all(np.diff(v[:0x7F]) > 0)         # magnitudes increase with the code
    np.testing.assert_array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def test_code_values_match_torch_float8():
    v = F.value_table()
    t = _torch_values(np.arange(256))
    np.testing.assert_array_equal(np.isnan(v), np.isnan(t))
    ok = ~np.isnan(v)
    np.testing.assert_array_equal(v[ok], t[ok])
    np.testing.assert_array_equal(np.signbit(v[ok]), np.signbit(t[ok]))


# ---- quantizer --------------------------------------------------------------

@pytest.mark.parametrize("s", [1.0, 0.5, 3.0, 2.0 ** -10, 0.0371])
def test_quantize_round_trip_every_code(s):
    v = F.value_table()
    for c in range(256):
        if np.isnan(v[c]):
            continue
        assert F.quantize_one(v[c] * s, s) == c, hex(c)


def test_quantize_midpoints_go_to_even_codes():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39); 1.1875 between 0x39 and 1.25 (0x3A)
    assert F.quantize_one(1.0625, 1.0) == 0x38
    assert F.quantize_one(1.1875, 1.0) == 0x3A
    assert F.quantize_one(-1.0625, 1.0) == 0xB8
    assert F.quantize_one(np.nextafter(1.0625, 2.0), 1.0) == 0x39
    assert F.quantize_one(np.nextafter(1.0625, 0.0), 1.0) == 0x38
    # subnormal range: 2^-10 is halfway between 0 and 2^-9, 3 * 2^-10 between 2^-9 and 2^-8
    assert F.quantize_one(2.0 ** -10, 1.0) == 0x00
    assert F.quantize_one(3 * 2.0 ** -10, 1.0) == 0x02
    assert F.quantize_one(-(2.0 ** -12), 1.0) == 0x80
    # the boundary between subnormals and normals: 7.5 * 2^-9 is halfway between 0x07 and 0x08
    assert F.quantize_one(7.5 * 2.0 ** -9, 1.0) == 0x08
    # midpoint at the top: 432 is halfway between 416 (0x7D) and 448 (0x7E)
    assert F.quantize_one(432.0, 1.0) == 0x7E
    assert F.quantize_one(424.0, 1.0) == 0x7D


def test_quantize_saturates_and_flags_nan():
    for x in [448.0, 460.0, 464.0, 1e6, float("inf")]:
        assert F.quantize_one(x, 1.0) == 0x7E
        assert F.quantize_one(-x, 1.0) == 0xFE
    assert F.quantize_one(float("nan"), 1.0) == 0x7F
    for s in [0.0, -1.0, float("inf"), float("nan")]:
        assert F.quantize_one(1.0, s) == 0x7F
    assert F.quantize_one(0.0, 1.0) == 0x00 and F.quantize_one(-0.0, 1.0) == 0x80


def test_quantize_matches_torch_rne_in_range():
    """PyTorch's fp32 -> float8_e4m3fn conversion rounds to nearest even; with s = 1 the quotient is x itself."""
    g = np.random.default_rng(7)
    x = np.concatenate([g.normal(0.0, 1.0, 4000) * 10.0 ** g.uniform(-3, 2.4, 4000),
                        g.uniform(-440, 440, 2000)]).astype(np.float32)
    # exact midpoints and their neighbours in every binade
    mids = (F.value_table()[1:0x7E] + F.value_table()[2:0x7F]) / 2.0
    x = np.concatenate([x, mids.astype(np.float32), np.nextafter(mids.astype(np.float32), np.float32(0))])
    x = x[np.abs(x) < 448.0]
    ours = F.quantize(x.astype(np.float64), 1.0)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_quantize_decision_is_the_exact_quotients():
    """The fp64 quotient decides as the exact rational x / s does (bf16 x, fp32 s)."""
    rng = random.Random(11)
    v = F.value_table()
    mags = [Fraction(float(m)) for m in v[:0x7F]]
    for _ in range(3000):
        x = float(torch.tensor(rng.gauss(0.0, 1.0) * 10 ** rng.uniform(-2, 2)).to(torch.bfloat16))
        s = float(np.float32(10 ** rng.uniform(-3, 1)))
        if rng.random() < 0.3:  # land exactly on a midpoint scaled by s
            c = rng.randrange(0, 0x7E)
            x = float(np.float32((v[c] + v[c + 1]) / 2 * 2.0 ** rng.randrange(-3, 4)))
            s = 2.0 ** rng.randrange(-3, 4)
        y = abs(Fraction(x)) / Fraction(s)
        if y >= 448:
            want = 0x7E
        else:
            d = [abs(m - y) for m in mags]
            best = min(d)
            cands = [c for c, dc in enumerate(d) if dc == best]
            want = cands[0] if len(cands) == 1 else next(c for c in cands if c % 2 == 0)
        want |= 0x80 if math.copysign(1.0, x) < 0 else 0
        assert F.quantize_one(x, s) == want, (x, s)


# ---- storage rules ------------------------------------------------------------

def test_append_writes_codes_under_the_destination_scale():
    nb, hkv, bs, d = 5, 2, 4, 8
    kc = np.full((nb, hkv, bs, d), 0x55, np.uint8)
    vc = np.full((nb, hkv, bs, d), 0x55, np.uint8)
    ks = np.arange(1, nb * hkv + 1, dtype=np.float64).reshape(nb, hkv) * 0.25
    vs = ks[::-1].copy()
    g = np.random.default_rng(3)
    kn = g.normal(size=(3, hkv, d))
    vn = g.normal(size=(3, hkv, d))
    slots = [2 * bs + 1, -1, 4 * bs + 3]
    F.append_kv(kc, vc, ks, vs, kn, vn, slots)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        pb, off = divmod(slot, bs)
        for j in range(hkv):
            want_k = [F.quantize_one(x, ks[pb, j]) for x in kn[t, j]]
            want_v = [F.quantize_one(x, vs[pb, j]) for x in vn[t, j]]
            assert kc[pb, j, off].tolist() == want_k and vc[pb, j, off].tolist() == want_v
    touched = np.zeros((nb, bs), bool)
    touched[2, 1] = touched[4, 3] = True
    kt, vt = kc.transpose(0, 2, 1, 3), vc.transpose(0, 2, 1, 3)  # [nb][B][Hkv][d]
    assert np.all(kt[~touched] == 0x55) and np.all(vt[~touched] == 0x55)
    # dequantized values are within half a step of the input
    deq = F.dequantize(kc, ks)
    step = np.abs(deq[2, 0, 1]) * 2.0 ** -4 + 2.0 ** -10 * ks[2, 0]
    assert np.all(np.abs(deq[2, 0, 1] - kn[0, 0]) <= step + 1e-12)


def test_append_skips_slots_outside_the_pool():
    kc = np.zeros((2, 1, 4, 4), np.uint8)
    vc = np.zeros((2, 1, 4, 4), np.uint8)
    s = np.ones((2, 1))
    F.append_kv(kc, vc, s, s, np.ones((2, 1, 4)), np.ones((2, 1, 4)), [8, 100])
    assert not kc.any() and not vc.any()


def test_copy_blocks_clones_codes_and_scales():
    g = np.random.default_rng(5)
    kc = g.integers(0, 256, (6, 2, 4, 8), dtype=np.uint8)
    vc = g.integers(0, 256, (6, 2, 4, 8), dtype=np.uint8)
    ks = g.uniform(0.1, 1, (6, 2))
    vs = g.uniform(0.1, 1, (6, 2))
    k0, v0, ks0, vs0 = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    F.copy_blocks(kc, vc, ks, vs, [(1, 4), (3, 0)])
    for src, dst in [(1, 4), (3, 0)]:
        assert np.array_equal(kc[dst], k0[src]) and np.array_equal(vc[dst], v0[src])
        assert np.array_equal(ks[dst], ks0[src]) and np.array_equal(vs[dst], vs0[src])
    for b in [1, 2, 3, 5]:
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(ks[b], ks0[b])


# ---- decode -------------------------------------------------------------------

def _random_cache(g, nb, hkv, bs, d):
    codes_k = g.integers(0, 256, (nb, hkv, bs, d), dtype=np.uint8)
    codes_v = g.integers(0, 256, (nb, hkv, bs, d), dtype=np.uint8)
    for c in (codes_k, codes_v):  # no NaN codes in stored tokens
        c[(c & 0x7F) == 0x7F] = 0x3C
        c &= 0xBF  # magnitudes below 2 (exponent field <= 7) keep the scores moderate
    return codes_k, codes_v, g.uniform(0.05, 0.5, (nb, hkv)), g.uniform(0.05, 0.5, (nb, hkv))


def test_decode_equals_dense_attention_over_tokenwise_dequantized_kv():
    g = np.random.default_rng(9)
    nb, hkv, hq, bs, d = 12, 2, 6, 4, 8
    kc, vc, ks, vs = _random_cache(g, nb, hkv, bs, d)
    lens = [9, 1, 0, 16]
    perm = g.permutation(nb)
    tables = np.zeros((len(lens), 4), np.int64)
    nxt = 0
    for n, s in enumerate(lens):
        for b in range(-(-s // bs)):
            tables[n, b] = perm[nxt]
            nxt += 1
    q = g.normal(size=(len(lens), hq, d))
    out = F.paged_decode(q, kc, vc, ks, vs, tables, lens, 0.35)
    for n, s in enumerate(lens):
        K = np.zeros((s, hkv, d))
        V = np.zeros((s, hkv, d))
        for t in range(s):
            pb, off = tables[n, t // bs], t % bs
            for j in range(hkv):
                K[t, j] = _torch_values(kc[pb, j, off]) * ks[pb, j]
                V[t, j] = _torch_values(vc[pb, j, off]) * vs[pb, j]
        np.testing.assert_allclose(out[n], A.dense_attention(q[n], K, V, 0.35), rtol=1e-12, atol=1e-14)


def test_decode_invariant_under_block_placement_with_scales():
    """Moving blocks (codes and scales together) to other physical ids changes nothing."""
    g = np.random.default_rng(13)
    nb, hkv, hq, bs, d = 10, 1, 2, 4, 8
    kc, vc, ks, vs = _random_cache(g, nb, hkv, bs, d)
    tables = np.array([[3, 7, 1]])
    q = g.normal(size=(1, hq, d))
    ref = F.paged_decode(q, kc, vc, ks, vs, tables, [11], 0.5)
    p = g.permutation(nb)
    inv = np.argsort(p)
    moved = F.paged_decode(q, kc[p], vc[p], ks[p], vs[p], inv[tables], [11], 0.5)
    np.testing.assert_allclose(moved, ref, rtol=1e-13, atol=1e-15)
    # the scale belongs to the block: moving codes without their scales does change the result
    wrong = F.paged_decode(q, kc[p], vc[p], ks, vs, inv[tables], [11], 0.5)
    assert not np.allclose(wrong, ref)

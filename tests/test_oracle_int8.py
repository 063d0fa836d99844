"""Pins for oracle/int8.py: the code values, the quantizer, the storage rules and the decode.

The code values are checked against NumPy's two's complement view of the
bytes (a library routine independent of the oracle); the quantizer's fp64
decision against exact rational arithmetic (Python's Fraction rounds half to
even); the decode against the separately written dense attention over K/V
dequantized token by token, and against a case whose answer is a plain mean.
"""

import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import int8 as I


def _np_values(codes):
    return np.asarray(codes, dtype=np.uint8).view(np.int8).astype(np.float64)


# ---- code values --------------------------------------------------------------

def test_code_values_are_twos_complement():
    v = I.value_table()
    np.testing.assert_array_equal(v, _np_values(np.arange(256)))
    assert v[0x00] == 0 and v[0x7F] == 127 and v[0x80] == -128 and v[0x81] == -127 and v[0xFF] == -1


# ---- quantizer --------------------------------------------------------------

@pytest.mark.parametrize("s", [1.0, 0.5, 3.0, 2.0 ** -10, 0.0371])
def test_quantize_round_trip_every_code(s):
    for c in range(-127, 128):
        assert I.code_value(I.quantize_one(c * s, s)) == c, c


def test_quantize_half_integers_go_to_even_codes():
    s = 0.25  # every k / 2 * s is exact
    for k2 in range(-253, 254, 2):  # odd multiples of 1/2: -126.5 .. 126.5
        y = k2 / 2
        want = math.floor(y) if math.floor(y) % 2 == 0 else math.floor(y) + 1
        assert I.code_value(I.quantize_one(y * s, s)) == want, y
    assert I.code_value(I.quantize_one(0.5, 1.0)) == 0
    assert I.code_value(I.quantize_one(-0.5, 1.0)) == 0
    assert I.code_value(I.quantize_one(1.5, 1.0)) == 2
    assert I.code_value(I.quantize_one(-2.5, 1.0)) == -2


def test_quantize_saturates_and_maps_nan_and_bad_scales_to_zero():
    assert I.code_value(I.quantize_one(127.4, 1.0)) == 127
    assert I.code_value(I.quantize_one(127.5, 1.0)) == 127
    assert I.code_value(I.quantize_one(-127.5, 1.0)) == -127
    assert I.code_value(I.quantize_one(1e30, 1e-3)) == 127
    assert I.code_value(I.quantize_one(-math.inf, 1.0)) == -127
    assert I.code_value(I.quantize_one(math.inf, 1.0)) == 127
    assert I.quantize_one(-0.0, 1.0) == 0 and I.quantize_one(1e-30, 1.0) == 0
    assert I.quantize_one(math.nan, 1.0) == 0
    for bad in (0.0, -1.0, math.inf, math.nan, -0.0):
        assert I.quantize_one(3.0, bad) == 0


def test_quantize_decision_is_the_exact_quotients():
    """The fp64 quotient decides as the exact rational x / s does (bf16 or fp32 x, fp32 s)."""
    rng = random.Random(17)
    for i in range(4000):
        x = rng.gauss(0.0, 1.0) * 10 ** rng.uniform(-2, 2.5)
        x = float(torch.tensor(x).to(torch.bfloat16)) if i % 2 else float(np.float32(x))
        s = float(np.float32(10 ** rng.uniform(-3, 1)))
        if rng.random() < 0.3:  # land exactly on a half-integer multiple of s
            s = 2.0 ** rng.randrange(-6, 3)
            x = (rng.randrange(-300, 300) + 0.5) * s
        y = Fraction(x) / Fraction(s)
        want = 127 if y >= 127 else (-127 if y <= -127 else round(y))
        assert I.code_value(I.quantize_one(x, s)) == want, (x, s)


def test_dequantized_value_within_half_a_step():
    g = np.random.default_rng(2)
    s = 0.013
    x = g.uniform(-127 * s, 127 * s, 2000)
    back = I.dequantize(I.quantize(x, s).reshape(1, 1, 1, -1), np.array([[s]]))[0, 0, 0]
    assert np.all(np.abs(back - x) <= s / 2 * (1 + 1e-12))


# ---- storage rules ------------------------------------------------------------

def test_append_writes_codes_under_the_destination_scale():
    nb, hkv, bs, d = 5, 2, 4, 8
    kc = np.full((nb, hkv, bs, d), 0x55, np.uint8)
    vc = np.full((nb, hkv, bs, d), 0x55, np.uint8)
    ks = np.arange(1, nb * hkv + 1, dtype=np.float64).reshape(nb, hkv) * 0.01
    vs = ks[::-1].copy()
    g = np.random.default_rng(3)
    kn = g.normal(size=(3, hkv, d))
    vn = g.normal(size=(3, hkv, d))
    slots = [2 * bs + 1, -1, 4 * bs + 3]
    I.append_kv(kc, vc, ks, vs, kn, vn, slots)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        pb, off = divmod(slot, bs)
        for j in range(hkv):
            want_k = [I.quantize_one(x, ks[pb, j]) for x in kn[t, j]]
            want_v = [I.quantize_one(x, vs[pb, j]) for x in vn[t, j]]
            assert kc[pb, j, off].tolist() == want_k and vc[pb, j, off].tolist() == want_v
    touched = np.zeros((nb, bs), bool)
    touched[2, 1] = touched[4, 3] = True
    kt, vt = kc.transpose(0, 2, 1, 3), vc.transpose(0, 2, 1, 3)  # [nb][B][Hkv][d]
    assert np.all(kt[~touched] == 0x55) and np.all(vt[~touched] == 0x55)


def test_append_skips_slots_outside_the_pool():
    kc = np.zeros((2, 1, 4, 4), np.uint8)
    vc = np.zeros((2, 1, 4, 4), np.uint8)
    s = np.ones((2, 1))
    I.append_kv(kc, vc, s, s, np.ones((2, 1, 4)), np.ones((2, 1, 4)), [8, 100])
    assert not kc.any() and not vc.any()


def test_copy_blocks_clones_codes_and_scales():
    g = np.random.default_rng(5)
    kc = g.integers(0, 256, (6, 2, 4, 8), dtype=np.uint8)
    vc = g.integers(0, 256, (6, 2, 4, 8), dtype=np.uint8)
    ks = g.uniform(0.1, 1, (6, 2))
    vs = g.uniform(0.1, 1, (6, 2))
    k0, v0, ks0, vs0 = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    I.copy_blocks(kc, vc, ks, vs, [(1, 4), (3, 0)])
    for src, dst in [(1, 4), (3, 0)]:
        assert np.array_equal(kc[dst], k0[src]) and np.array_equal(vc[dst], v0[src])
        assert np.array_equal(ks[dst], ks0[src]) and np.array_equal(vs[dst], vs0[src])
    for b in [1, 2, 3, 5]:
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(ks[b], ks0[b])


# ---- decode -------------------------------------------------------------------

def _random_cache(g, nb, hkv, bs, d):
    codes_k = g.integers(0, 256, (nb, hkv, bs, d), dtype=np.uint8)
    codes_v = g.integers(0, 256, (nb, hkv, bs, d), dtype=np.uint8)
    return codes_k, codes_v, g.uniform(0.002, 0.02, (nb, hkv)), g.uniform(0.002, 0.02, (nb, hkv))


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
    out = I.paged_decode(q, kc, vc, ks, vs, tables, lens, 0.35)
    for n, s in enumerate(lens):
        K = np.zeros((s, hkv, d))
        V = np.zeros((s, hkv, d))
        for t in range(s):
            pb, off = tables[n, t // bs], t % bs
            for j in range(hkv):
                K[t, j] = _np_values(kc[pb, j, off]) * ks[pb, j]
                V[t, j] = _np_values(vc[pb, j, off]) * vs[pb, j]
        np.testing.assert_allclose(out[n], A.dense_attention(q[n], K, V, 0.35), rtol=1e-12, atol=1e-14)


def test_decode_of_equal_keys_is_the_mean_of_the_values():
    """All key codes 0: every score is 0, the weights are equal, the output is the mean of the stored values."""
    kc = np.zeros((2, 1, 2, 2), np.uint8)
    vc = np.zeros((2, 1, 2, 2), np.uint8)
    vc[1, 0, 0] = np.array([10, -20], np.int8).view(np.uint8)   # token 0 (block 1)
    vc[1, 0, 1] = np.array([30, 40], np.int8).view(np.uint8)    # token 1
    vc[0, 0, 0] = np.array([-2, 127], np.int8).view(np.uint8)   # token 2 (block 0)
    ks = np.ones((2, 1))
    vs = np.array([[0.25], [0.5]])
    out = I.paged_decode(np.array([[[1.0, -3.0]]]), kc, vc, ks, vs, np.array([[1, 0]]), [3], 0.7)
    # values: [5, -10], [15, 20], [-0.5, 31.75]
    np.testing.assert_allclose(out[0, 0], [(5 + 15 - 0.5) / 3, (-10 + 20 + 31.75) / 3], rtol=1e-15)


def test_decode_invariant_under_block_placement_with_scales():
    """Moving blocks (codes and scales together) to other physical ids changes nothing."""
    g = np.random.default_rng(13)
    nb, hkv, hq, bs, d = 10, 1, 2, 4, 8
    kc, vc, ks, vs = _random_cache(g, nb, hkv, bs, d)
    tables = np.array([[3, 7, 1]])
    q = g.normal(size=(1, hq, d))
    ref = I.paged_decode(q, kc, vc, ks, vs, tables, [11], 0.5)
    p = g.permutation(nb)
    inv = np.argsort(p)
    moved = I.paged_decode(q, kc[p], vc[p], ks[p], vs[p], inv[tables], [11], 0.5)
    np.testing.assert_allclose(moved, ref, rtol=1e-13, atol=1e-15)
    wrong = I.paged_decode(q, kc[p], vc[p], ks, vs, inv[tables], [11], 0.5)
    assert not np.allclose(wrong, ref)

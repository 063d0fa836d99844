"""Pins for oracle/attention.py: page-printed values, closed forms, special cases, invariants."""

import math

import numpy as np
import pytest

from conftest import golden
from oracle import attention as A

SYM = {"0": 0.0, "1": 1.0, "-1": -1.0, "sqrt2": math.sqrt(2.0), "1/sqrt2": 1.0 / math.sqrt(2.0),
       "ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0)}


def _num(x):
    return SYM[x] if isinstance(x, str) else float(x)


def _p2():
    g = golden("p2_two_page_attention.json")
    q = np.array([_num(x) for x in g["q"]])
    K = np.array([[_num(x) for x in row] for row in g["K"]])
    V = np.array(g["V"], dtype=np.float64)
    return g, q, K, V, _num(g["scale"])


def test_p2_scores_and_weights():
    g, q, K, V, scale = _p2()
    s = scale * (K @ q)
    np.testing.assert_allclose(s, [_num(x) for x in g["scores"]], atol=1e-15)
    np.testing.assert_allclose(np.exp(s), g["exp_scores"], rtol=1e-14)
    np.testing.assert_allclose(A.attention_weights(q, K, scale), g["weights"], atol=1e-15)


def test_p2_contiguous_output():
    g, q, K, V, scale = _p2()
    np.testing.assert_allclose(A.softmax_attention(q, K, V, scale), g["output"], atol=1e-14)
    out = A.dense_attention(q[None, :], K[:, None, :], V[:, None, :], scale)
    np.testing.assert_allclose(out[0], g["output"], atol=1e-14)


def test_p2_paged_output_two_pages():
    """Two tokens per page, logical pages in physical blocks 9 and 2."""
    g, q, K, V, scale = _p2()
    table = g["paged"]["block_table"]
    nb = 10
    kp = np.full((nb, 1, 2, 2), np.nan)
    vp = np.full((nb, 1, 2, 2), np.nan)
    for t in range(4):
        lb, off, pb, _ = A.translate(t, 2, table)
        kp[pb, 0, off] = K[t]
        vp[pb, 0, off] = V[t]
    out = A.paged_decode(q[None, None, :], kp, vp, np.array([table]), [4], scale)
    np.testing.assert_allclose(out[0, 0], g["output"], atol=1e-14)


def test_p2_page_sums_and_stable_merge():
    g, q, K, V, scale = _p2()
    s = scale * (K @ q)
    pa, pb = g["paged"]["page_A"], g["paged"]["page_B"]
    Za, Na = A.page_sums(s[:2], V[:2])
    Zb, Nb = A.page_sums(s[2:], V[2:])
    assert Za == pytest.approx(pa["Z"], abs=1e-14) and Zb == pytest.approx(pb["Z"], abs=1e-13)
    np.testing.assert_allclose(Na, pa["N"], atol=1e-14)
    np.testing.assert_allclose(Nb, pb["N"], atol=1e-13)
    np.testing.assert_allclose((Na + Nb) / (Za + Zb), g["output"], atol=1e-14)
    ma, za, ua = A.block_summary(s[:2], V[:2])
    mb, zb, ub = A.block_summary(s[2:], V[2:])
    assert ma == pytest.approx(_num(pa["m"]), abs=1e-15) and za == pytest.approx(pa["z"], abs=1e-15)
    assert mb == pytest.approx(_num(pb["m"]), abs=1e-15) and zb == pytest.approx(pb["z"], abs=1e-15)
    np.testing.assert_allclose(ua, pa["u"], atol=1e-15)
    np.testing.assert_allclose(ub, pb["u"], atol=1e-15)
    m, z, u = A.merge_summaries([(ma, za, ua), (mb, zb, ub)])
    mg = g["paged"]["merged"]
    assert m == pytest.approx(_num(mg["m"]), abs=1e-15) and z == pytest.approx(mg["z"], abs=1e-15)
    np.testing.assert_allclose(u, mg["u"], atol=1e-14)
    np.testing.assert_allclose(u / z, mg["output"], atol=1e-14)
    # merge order does not matter
    m2, z2, u2 = A.merge_summaries([(mb, zb, ub), (ma, za, ua)])
    np.testing.assert_allclose(u2 / z2, mg["output"], atol=1e-14)


def test_teaching_t3_paged_equals_dense_with_junk_tail():
    """[P1] section 20 test 3: table [2, 0], junk in the masked tail, paged == dense."""
    t3 = golden("block_manager_traces.json")["teaching_tests"]["t3"]
    B = t3["block_size"]
    pop_order = list(reversed(t3["free_stack"]))
    kv = np.array(t3["kv"])
    S = len(kv)
    table = pop_order[: -(-S // B)]
    assert table == t3["expect_table"]
    kp = np.zeros((t3["num_blocks"], 1, B, 1))
    vp = np.zeros((t3["num_blocks"], 1, B, 1))
    for t in range(S):
        _, off, pb, _ = A.translate(t, B, table)
        kp[pb, 0, off, 0], vp[pb, 0, off, 0] = kv[t]
    tail = table[-1]
    for off, (k, v) in t3["junk"].items():
        kp[tail, 0, int(off), 0], vp[tail, 0, int(off), 0] = k, v
    q = np.array([[[t3["q"]]]])
    paged = A.paged_decode(q, kp, vp, np.array([table]), [S], t3["scale"])[0, 0, 0]
    dense = A.dense_attention(q[0], kv[:, 0][:, None, None], kv[:, 1][:, None, None], t3["scale"])[0, 0]
    assert paged == pytest.approx(dense, rel=1e-14)
    # the junk would change the answer if it were read
    with_junk = A.dense_attention(q[0], np.array([999.0, 888.0] + list(kv[:, 0]))[:, None, None],
                                  np.array([-999.0, -888.0] + list(kv[:, 1]))[:, None, None], t3["scale"])[0, 0]
    assert abs(with_junk - paged) > 1.0


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, 16))
    v = rng.standard_normal((1, 16))
    q = rng.standard_normal(16)
    assert np.array_equal(A.softmax_attention(q, k, v, 0.25), v[0])


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    k = np.tile(rng.standard_normal(8), (37, 1))
    v = rng.standard_normal((37, 8))
    q = rng.standard_normal(8)
    np.testing.assert_allclose(A.softmax_attention(q, k, v, 0.3), v.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_two_tokens_logistic_closed_form():
    """softmax over two scores is a logistic: o = v0 + (v1 - v0) / (1 + exp(s0 - s1))."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        k = rng.standard_normal((2, 5))
        v = rng.standard_normal((2, 5))
        q = rng.standard_normal(5)
        scale = 0.7
        s0, s1 = scale * float(k[0] @ q), scale * float(k[1] @ q)
        expect = v[0] + (v[1] - v[0]) / (1.0 + math.exp(s0 - s1))
        np.testing.assert_allclose(A.softmax_attention(q, k, v, scale), expect, rtol=1e-12, atol=1e-14)


def test_large_scores_stay_finite_and_dominant_token_wins():
    k = np.zeros((5, 2))
    k[3] = [1000.0, 0.0]
    k[1] = [-1000.0, 0.0]
    v = np.arange(10, dtype=np.float64).reshape(5, 2)
    out = A.softmax_attention(np.array([1.0, 0.0]), k, v, 1.0)
    assert np.all(np.isfinite(out))
    assert np.array_equal(out, v[3])  # exp(-1000) underflows to exactly 0


def test_weights_sum_to_one():
    rng = np.random.default_rng(4)
    for s in (1, 2, 17, 300):
        w = A.attention_weights(rng.standard_normal(32), rng.standard_normal((s, 32)) * 3, 0.5)
        assert abs(w.sum() - 1.0) < 1e-14
        assert np.all(w >= 0)


def _random_paged(rng, n_seqs, hq, hkv, d, B, lens, nb, perm=None):
    k_log = [rng.standard_normal((L, hkv, d)) for L in lens]
    v_log = [rng.standard_normal((L, hkv, d)) for L in lens]
    kp = np.full((nb, hkv, B, d), np.nan)
    vp = np.full((nb, hkv, B, d), np.nan)
    order = list(perm if perm is not None else rng.permutation(nb))
    max_blocks = max(-(-L // B) for L in lens)
    tables = np.zeros((n_seqs, max_blocks), dtype=np.int64)
    it = iter(order)
    for n, L in enumerate(lens):
        for b in range(-(-L // B)):
            tables[n, b] = next(it)
        for t in range(L):
            _, off, pb, _ = A.translate(t, B, tables[n])
            kp[pb, :, off] = k_log[n][t]
            vp[pb, :, off] = v_log[n][t]
    q = rng.standard_normal((n_seqs, hq, d))
    return q, kp, vp, tables, k_log, v_log


def test_paged_equals_contiguous_dense_random():
    rng = np.random.default_rng(5)
    lens = [1, 15, 16, 17, 33, 64, 100]
    q, kp, vp, tables, k_log, v_log = _random_paged(rng, len(lens), 8, 2, 16, 16, lens, 40)
    out = A.paged_decode(q, kp, vp, tables, lens, 0.25)
    for n in range(len(lens)):
        dense = A.dense_attention(q[n], k_log[n], v_log[n], 0.25)
        np.testing.assert_allclose(out[n], dense, rtol=1e-12, atol=1e-14)
        assert np.all(np.isfinite(out[n]))  # NaN-filled tails and free blocks never read


def test_placement_invariance_bit_identical():
    """Moving blocks to other physical ids (and rewriting the tables) leaves the output bit-identical."""
    rng = np.random.default_rng(6)
    lens = [5, 16, 40, 71]
    q, kp, vp, tables, _, _ = _random_paged(rng, 4, 4, 4, 8, 8, lens, 24)
    out1 = A.paged_decode(q, kp, vp, tables, lens, 0.5)
    perm = rng.permutation(24)  # new id of old block b is perm[b]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    out2 = A.paged_decode(q, kp2, vp2, perm[tables], lens, 0.5)
    assert np.array_equal(out1, out2)


def test_gqa_head_mapping_consecutive_heads_share():
    """Query head h reads KV head h // (Hq/Hkv): with constant values per KV head the output is that constant."""
    rng = np.random.default_rng(7)
    hq, hkv, d, B, L = 8, 2, 4, 4, 10
    kp = rng.standard_normal((3, hkv, B, d))
    vp = np.zeros((3, hkv, B, d))
    vp[:, 0] = 3.0
    vp[:, 1] = -5.0
    out = A.paged_decode(rng.standard_normal((1, hq, d)), kp, vp, np.array([[2, 0, 1]]), [L], 1.0)
    expect = np.array([3.0] * 4 + [-5.0] * 4)
    np.testing.assert_allclose(out[0, :, 0], expect, rtol=1e-15)


def test_mha_and_mqa_reduce_to_per_head_attention():
    rng = np.random.default_rng(8)
    d, B, L = 8, 4, 9
    for hq, hkv in ((4, 4), (4, 1)):
        q, kp, vp, tables, k_log, v_log = _random_paged(rng, 1, hq, hkv, d, B, [L], 6)
        out = A.paged_decode(q, kp, vp, tables, [L], 0.35)
        for h in range(hq):
            j = h // (hq // hkv)
            np.testing.assert_allclose(out[0, h], A.softmax_attention(q[0, h], k_log[0][:, j], v_log[0][:, j], 0.35),
                                       rtol=1e-13)


def test_zero_length_sequence_gives_zeros():
    kp = np.full((2, 1, 4, 3), np.nan)
    out = A.paged_decode(np.ones((1, 2, 3)), kp, kp, np.zeros((1, 1), dtype=int), [0], 1.0)
    assert np.array_equal(out, np.zeros((1, 2, 3)))


def test_translation_pins():
    for c in golden("translation.json")["cases"]:
        table = c.get("block_table", [0] * 8)
        lb, off, pb, slot = A.translate(c["token"], c["block_size"], table)
        e = c["expect"]
        assert (lb, off) == (e["logical_block"], e["offset"]), c["source"]
        if "physical_block" in e:
            assert pb == e["physical_block"], c["source"]
        if "slot" in e:
            assert slot == e["slot"], c["source"]


def test_translation_exhaustive_small():
    """Every token lands in exactly one slot; slots of distinct tokens differ; offsets stay below B."""
    for B in (1, 3, 8, 16):
        table = [5, 0, 7, 2, 9]
        seen = set()
        for t in range(len(table) * B):
            lb, off, pb, slot = A.translate(t, B, table)
            assert 0 <= off < B and lb * B + off == t and pb == table[lb]
            assert slot not in seen
            seen.add(slot)


def test_append_writes_only_the_target_slot():
    """[P1] section 16: position 35 of sequence A (table [10, 11, 13]) lands in block 13 at offset 3."""
    B, hkv, d = 16, 2, 4
    kp = np.zeros((16, hkv, B, d))
    vp = np.zeros((16, hkv, B, d))
    _, _, _, slot = A.translate(35, B, [10, 11, 13])
    kn = np.arange(hkv * d, dtype=np.float64).reshape(1, hkv, d) + 1
    A.append_kv(kp, vp, kn, -kn, [slot])
    assert np.array_equal(kp[13, :, 3], kn[0]) and np.array_equal(vp[13, :, 3], -kn[0])
    kp[13, :, 3] = 0
    vp[13, :, 3] = 0
    assert not kp.any() and not vp.any()
    A.append_kv(kp, vp, kn, kn, [-1])  # negative slot: skipped
    assert not kp.any()


def test_copy_blocks_clones_whole_block():
    rng = np.random.default_rng(9)
    kp = rng.standard_normal((3, 6, 2, 4, 5))  # with a layer axis
    vp = rng.standard_normal((3, 6, 2, 4, 5))
    k0, v0 = kp.copy(), vp.copy()
    A.copy_blocks(kp, vp, [(1, 4), (2, 0)])
    assert np.array_equal(kp[:, 4], k0[:, 1]) and np.array_equal(vp[:, 0], v0[:, 2])
    untouched = [1, 2, 3, 5]
    assert np.array_equal(kp[:, untouched], k0[:, untouched])

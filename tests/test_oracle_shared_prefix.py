"""Pins for the shared-prefix grouping rule (oracle/block_manager.shared_prefix_groups)
and for the decomposition a shared-prefix decode relies on.

A decode may read a full block shared by several sequences once for all of
them ([P1] section 15 item 1: full shared blocks are immutable and readable by
all sharers at once) and merge that part of each sequence's attention with the
part over its own blocks ([P2] section 11).  The grouping rule only chooses
which rows are read together; the attention it must reproduce is the plain
paged decode of the oracle.
"""

import random

import numpy as np
import pytest

import synth
from conftest import golden
from oracle import attention as A
from oracle import block_manager as BM


def _batch(m, seqs):
    return [list(m.tables[s]) for s in seqs], [m.lens[s] for s in seqs]


def test_fork_35_trace_shares_two_full_blocks():
    """[P1] sections 14-17: after the fork and after both appends, A and B share blocks 10 and 11 (32 tokens)."""
    g = golden("block_manager_traces.json")["fork_35"]
    B, nb = g["block_size"], g["num_blocks"]
    order = g["pop_order_prefix"] + [b for b in range(nb) if b not in g["pop_order_prefix"]]
    m = BM.BlockManagerModel(nb, B, order)
    assert m.add_seq("A", g["prompt"]) == BM.OK and m.fork("A", "B") == BM.OK
    # before the appends the 3-token tail block 12 is shared too, but it is not full
    tables, lens = _batch(m, ["A", "B"])
    assert tables == [[10, 11, 12], [10, 11, 12]]
    shared = g["after_step"]["shared_full_prefix_tokens"]
    assert BM.shared_prefix_groups(tables, lens, B, 8) == [(0, 2, shared)]
    assert m.append_slot("A")[0] == BM.OK and m.append_slot("B")[0] == BM.OK
    tables, lens = _batch(m, ["A", "B"])
    assert tables == [g["after_step"]["A"], g["after_step"]["B"]]
    assert BM.shared_prefix_groups(tables, lens, B, 8) == [(0, 2, shared)]
    # a group of one is no group
    assert BM.shared_prefix_groups(tables, lens, B, 1) == []


def test_exercise_2_shares_sixteen_tokens():
    """[P1] section 24: A = [0, 1, 3, 4] (32 tokens) and B = [0, 1, 2] (22 tokens) share blocks 0 and 1."""
    g = golden("block_manager_traces.json")["exercise_2"]
    f = g["final"]
    B = g["block_size"]
    groups = BM.shared_prefix_groups([f["A"], f["B"]], [f["len_A"], f["len_B"]], B, 8)
    assert groups == [(0, 2, f["shared_prefix_tokens"])]
    # the order of the rows does not matter for two rows
    assert BM.shared_prefix_groups([f["B"], f["A"]], [f["len_B"], f["len_A"]], B, 8) == groups


def test_parallel_sampling_workload_groups():
    """32 prompts of 2,055 tokens forked into 8 samples: one group of 8 per prompt, 128 full blocks shared."""
    w = synth.fork()
    P, S = synth.FORK_PROMPTS, synth.FORK_SAMPLES
    prompt = w.fixed_lens[0]
    nb = P * (-(-prompt // w.block_size)) + P * S * 2
    m = BM.BlockManagerModel(nb, w.block_size)
    for p in range(P):
        assert m.add_seq(p * S, prompt) == BM.OK
        for s in range(1, S):
            assert m.fork(p * S, p * S + s) == BM.OK
    seqs = list(range(P * S))
    shared = (prompt // w.block_size) * w.block_size
    assert shared == 2048
    for step in range(3):  # before and after the copy-on-write of the 7-token tails
        tables, lens = _batch(m, seqs)
        assert BM.shared_prefix_groups(tables, lens, w.block_size, 8) == [(p * S, S, shared) for p in range(P)]
        assert BM.shared_prefix_groups(tables, lens, w.block_size, 4) == [
            (p * S + h * 4, 4, shared) for p in range(P) for h in range(2)]
        assert m.append_slots(seqs)[0] == BM.OK


def test_join_keeps_the_bytes_saved():
    """A row that would shrink the shared part more than it adds starts a run of its own."""
    B = 4
    x = list(range(100, 110))
    tables = [x, list(x), [100] + list(range(200, 209)), [100] + list(range(200, 209))]
    lens = [40, 40, 40, 40]
    # rows 0-1 share 10 blocks; row 2 shares 1 with them: 2 * 1 < 1 * 10, so it does not join;
    # rows 2-3 share all 10 of theirs
    assert BM.shared_prefix_groups(tables, lens, B, 8) == [(0, 2, 40), (2, 2, 40)]
    # a row that shares at least half of a pair's blocks joins (2 * 5 >= 1 * 10)
    t3 = [x, list(x), x[:5] + list(range(300, 305))]
    assert BM.shared_prefix_groups(t3, [40, 40, 40], B, 8) == [(0, 3, 20)]
    # only full blocks of every member count: a 38-token row has 9 full blocks
    assert BM.shared_prefix_groups([x, list(x)], [40, 38], B, 8) == [(0, 2, 36)]
    # rows with no full block never group
    assert BM.shared_prefix_groups([x, list(x)], [3, 3], B, 8) == []


def _random_forest(rng, B, nb, min_len=1):
    m = BM.BlockManagerModel(nb, B, rng.sample(range(nb), nb))
    live = []
    nid = 0
    for _ in range(rng.randint(3, 7)):
        assert m.add_seq(nid, rng.randint(min_len, 12 * B)) == BM.OK
        live.append(nid)
        nid += 1
    if min_len >= B:  # at least one fork of a sequence that holds a full block
        assert m.fork(0, nid) == BM.OK
        live.append(nid)
        nid += 1
    for _ in range(rng.randint(5, 40)):
        op = rng.random()
        if op < 0.4:
            parent = rng.choice(live)
            assert m.fork(parent, nid) == BM.OK
            live.append(nid)
            nid += 1
        else:
            for _ in range(rng.randint(1, 2 * B)):
                assert m.append_slot(rng.choice(live))[0] == BM.OK
    return m, live


@pytest.mark.parametrize("seed", range(25))
def test_groups_are_valid_on_random_fork_forests(seed):
    """Invariants of any returned grouping, on random fork trees and batch orders."""
    rng = random.Random(seed)
    B = rng.choice([4, 8, 16])
    m, live = _random_forest(rng, B, 4096)
    order = list(live)
    if seed % 2:
        rng.shuffle(order)
    else:
        order.sort()
    tables, lens = _batch(m, order)
    cap = rng.choice([2, 3, 4, 8])
    groups = BM.shared_prefix_groups(tables, lens, B, cap)
    last_end = 0
    for first, count, shared in groups:
        assert first >= last_end and 2 <= count <= cap  # consecutive, disjoint, in order
        last_end = first + count
        assert shared > 0 and shared % B == 0
        nblk = shared // B
        for r in range(first, first + count):
            assert shared <= lens[r]
            assert tables[r][:nblk] == tables[first][:nblk]
        for b in tables[first][:nblk]:  # every shared block is referenced at least once per member
            assert m.ref[b] >= count
    # every adjacent pair of rows that shares a full block ends up in some group
    # unless a group boundary or the member cap intervened
    in_group = {r for f, c, _ in groups for r in range(f, f + c)}
    for r in range(len(order) - 1):
        if min(lens[r], lens[r + 1]) >= B and tables[r][0] == tables[r + 1][0]:
            assert r in in_group or r + 1 in in_group


@pytest.mark.parametrize("seed", range(6))
def test_prefix_and_suffix_summaries_merge_to_the_paged_decode(seed):
    """[P2] section 11 on a grouping: for every member, the summary over the group's shared
    tokens (read once, from the first member's table) merged with the summary over the
    member's remaining tokens equals the plain paged decode of that member."""
    rng = random.Random(100 + seed)
    B, hkv, g, d = 8, 2, 2, 16
    m, live = _random_forest(rng, B, 2048, min_len=2 * B)
    tables, lens = _batch(m, sorted(live))
    groups = BM.shared_prefix_groups(tables, lens, B, 4)
    assert groups
    nr = np.random.default_rng(seed)
    nb = m.num_blocks
    k_pool = nr.standard_normal((nb, hkv, B, d))
    v_pool = nr.standard_normal((nb, hkv, B, d))
    n = len(lens)
    q = nr.standard_normal((n, hkv * g, d))
    scale = 1 / np.sqrt(d)
    mb = max(len(t) for t in tables)
    tab = np.array([t + [0] * (mb - len(t)) for t in tables])
    plain = A.paged_decode(q, k_pool, v_pool, tab, lens, scale)
    for first, count, shared in groups:
        for r in range(first, first + count):
            for h in range(hkv * g):
                j = h // g
                ks = A.gather_sequence(k_pool, tables[first], shared, j)
                vs = A.gather_sequence(v_pool, tables[first], shared, j)
                kp = A.gather_sequence(k_pool, tables[r], lens[r], j)
                vp = A.gather_sequence(v_pool, tables[r], lens[r], j)
                parts = [A.block_summary(scale * ks @ q[r, h], vs)]
                if lens[r] > shared:
                    parts.append(A.block_summary(scale * kp[shared:] @ q[r, h], vp[shared:]))
                _, z, u = A.merge_summaries(parts)
                np.testing.assert_allclose(u / z, plain[r, h], rtol=1e-12, atol=1e-12)

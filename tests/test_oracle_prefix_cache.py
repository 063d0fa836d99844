"""Pins for the prefix-caching block manager model (oracle/block_manager.PrefixCachingModel).

The pages fix what a prefix cache must do ([P1] sections 18-19, [P2] section
6, [P3] "Prefix caching"); the readings that complete it are in the model's
docstring.  Every hit is also checked against brute force: the token prefix a
reused block stands for must equal the request's.
"""

import random

import pytest

from conftest import golden
from oracle import block_manager as BM


def _check(m):
    """Invariants: the pool splits into free, idle-cached and referenced blocks; references match the tables;
    cached blocks are full wherever they are used; the index and the entries agree."""
    refs = [0] * m.num_blocks
    for seq, t in m.tables.items():
        for lb, b in enumerate(t):
            refs[b] += 1
            if b in m.entry:
                assert (lb + 1) * m.block_size <= m.lens[seq], "a cached block must be full"
    assert refs == m.ref
    free, idle = set(m.free), set(m.idle)
    used = {b for b in range(m.num_blocks) if m.ref[b] > 0}
    assert len(free) == len(m.free) and len(idle) == len(m.idle)
    assert not (free & idle) and not (free & used) and not (idle & used)
    assert free | idle | used == set(range(m.num_blocks))
    assert idle <= set(m.entry) and not (free & set(m.entry))
    assert {b: k for k, b in m.index.items()} == m.entry
    for b, key in m.entry.items():  # a cached block holds the tokens of its chain in every table that uses it
        for seq, t in m.tables.items():
            toks = m.tokens[seq]
            if b in t and toks is not None:
                lb = t.index(b)
                assert tuple(toks[:(lb + 1) * m.block_size]) == key


def test_two_requests_reuse_the_first_two_blocks():
    g = golden("prefix_cache.json")["two_requests_same_prefix"]
    B = g["block_size"]
    m = BM.PrefixCachingModel(32, B)
    common = list(range(1, g["shared_token_ids"] + 1))
    assert m.add_seq_tokens("A", common + [100, 101, 102]) == (BM.OK, 0)
    st, hit = m.add_seq_tokens("B", common + [200, 201])
    assert st == BM.OK and hit == g["shared_full_blocks"] * B
    assert m.tables["A"][:2] == m.tables["B"][:2]
    assert m.tables["A"][2] != m.tables["B"][2]  # separate suffix blocks
    assert [m.ref[b] for b in m.tables["B"]] == [2, 2, 1]
    _check(m)


def test_equal_text_after_a_different_prefix_does_not_match():
    g = golden("prefix_cache.json")["context_matters"]
    B = g["block_size"]
    m = BM.PrefixCachingModel(32, B)
    assert m.add_seq_tokens("A", [1, 2, 3, 4, 5, 6, 7, 8])[0] == BM.OK
    # block 1's text again, after another first block
    st, hit = m.add_seq_tokens("C", [9, 9, 9, 9, 5, 6, 7, 8])
    assert st == BM.OK and hit == g["reused_blocks"] * B
    assert not set(m.tables["A"]) & set(m.tables["C"])
    # and the text of A's first block alone, at the start, does match
    assert m.add_seq_tokens("D", [1, 2, 3, 4, 0])[1] == B
    _check(m)


def test_released_blocks_stay_cached_and_are_revived():
    g = golden("prefix_cache.json")["revival"]
    m = BM.PrefixCachingModel(16, 4)
    toks = list(range(10, 22))  # 3 full blocks
    assert m.add_seq_tokens("A", toks) == (BM.OK, 0)
    blocks = list(m.tables["A"])
    assert m.free_seq("A") == BM.OK
    assert all(m.ref[b] == g["ref_after_release"] for b in blocks)
    assert set(m.idle) == set(blocks) and m.stats()["num_cached"] == 3
    st, hit = m.add_seq_tokens("A2", toks + [99])
    assert st == BM.OK and hit == 12 and m.tables["A2"][:3] == blocks
    assert all(m.ref[b] == g["ref_after_reuse"] for b in blocks) and not m.idle
    _check(m)


def test_finishing_one_sharer_frees_only_its_suffix():
    g = golden("prefix_cache.json")["finish_one_of_two"]
    B = g["block_size"]
    m = BM.PrefixCachingModel(32, B)
    common = list(range(1, 2 * B + 1))
    m.add_seq_tokens("A", common + [7, 7])
    m.add_seq_tokens("B", common + [8])
    shared = m.tables["A"][:g["shared_full_blocks"]]
    suffix_a = m.tables["A"][2]
    assert m.free_seq("A") == BM.OK
    assert [m.ref[b] for b in shared] == [g["refs_after_A_finishes"]] * 2  # B keeps its references
    # A's suffix block (partial, not cached) is what the next allocation gets
    assert m.add_seq_tokens("C", [50, 51])[0] == BM.OK and m.tables["C"] == [suffix_a]
    _check(m)


def test_rag_requests_reuse_the_document_blocks():
    g = golden("prefix_cache.json")["byte_identical"]
    B = g["block_size"]
    m = BM.PrefixCachingModel(256, B)
    doc = [random.Random(1).randrange(32000) for _ in range(5 * B + 3)]  # system prompt + document
    hits = []
    for i in range(6):
        st, hit = m.add_seq_tokens(i, doc + [1000 + i] * (3 + i))
        assert st == BM.OK
        hits.append(hit)
    assert hits == [0] + [5 * B] * 5  # the first request pays the full prefill
    # one token different in the first block: nothing matches
    bad = list(doc)
    bad[3] += 1
    assert m.add_seq_tokens("x", bad)[1] == 0
    _check(m)


def test_eviction_under_pressure_takes_the_least_recently_released():
    """[P1] section 19 / [P2] section 6: idle cached blocks are reclaimed (oldest release first) before an allocation
    fails; a running request's blocks are never taken; an evicted prefix misses later."""
    m = BM.PrefixCachingModel(8, 2)
    a, b = [1, 2, 3, 4], [5, 6, 7, 8]  # 2 full blocks each
    m.add_seq_tokens("A", a)
    m.add_seq_tokens("B", b)
    m.add_seq_tokens("R", [9, 9, 9, 9])  # running throughout
    a0, a1 = m.tables["A"]
    b0, b1 = m.tables["B"]
    r = list(m.tables["R"])
    m.free_seq("A")
    m.free_seq("B")
    # released from the last block to the first: a request's deepest block is its oldest idle entry
    assert m.idle == [a1, a0, b1, b0] and len(m.free) == 2
    assert m.add_seq_tokens("N", [20, 21, 22, 23, 24, 25]) == (BM.OK, 0)  # 3 blocks: 2 free + a1 evicted
    assert m.evictions == 1 and a1 in m.tables["N"]
    # A's first block survived: reused (0 -> 1); its second is recomputed in the oldest idle block, b1
    assert m.add_seq_tokens("A'", a) == (BM.OK, 2)
    assert m.tables["A'"] == [a0, b1] and m.evictions == 2
    # all 8 blocks are now held or idle-but-needed: B's request fails and changes nothing
    before = (list(m.free), list(m.idle), list(m.ref), dict(m.index))
    assert m.add_seq_tokens("B'", b)[0] == BM.ERR_NO_FREE_BLOCKS
    assert (list(m.free), list(m.idle), list(m.ref), dict(m.index)) == before
    assert m.tables["R"] == r  # the running request was never touched
    m.free_seq("N")
    assert m.add_seq_tokens("B'", b) == (BM.OK, 2)  # b0 survived, b1 did not
    _check(m)


def test_blocks_filled_by_generated_tokens_become_reusable():
    m = BM.PrefixCachingModel(32, 4)
    m.add_seq_tokens("A", [1, 2, 3, 4, 5, 6])
    for t in (7, 8, 9):
        assert m.append_token("A", t)[0] == BM.OK
    # block 1 = [5, 6, 7, 8] filled by two generated tokens: cached
    assert m.add_seq_tokens("B", [1, 2, 3, 4, 5, 6, 7, 8, 0])[1] == 8
    # an append without a token id ends A's chain: its next full block is not cached
    m2 = BM.PrefixCachingModel(32, 4)
    m2.add_seq_tokens("A", [1, 2, 3, 4, 5, 6])
    m2.append_token("A", None)
    m2.append_token("A", 8)
    assert m2.stats()["num_cached"] == 1
    # the same block produced twice (same prefix, same tokens) is cached once; the chain continues through it
    m3 = BM.PrefixCachingModel(32, 2)
    m3.add_seq_tokens("P", [1, 2, 3])
    assert m3.fork("P", "Q") == BM.OK
    for s in ("P", "Q"):
        m3.append_token(s, 4)   # [3, 4] completes block 1 in both (Q copied P's tail on write)
        m3.append_token(s, 5)
        m3.append_token(s, 6)   # [5, 6] completes block 2
    assert m3.stats()["num_cached"] == 3
    st, hit = m3.add_seq_tokens("R", [1, 2, 3, 4, 5, 6, 7])
    assert st == BM.OK and hit == 6
    _check(m3)


def test_a_miss_can_meet_a_cached_child_of_an_evicted_parent():
    """Chains are content.  Two forks that generate the same tokens cache [1..4] in one's block and [1..6] in the
    other's; after [1..4] is evicted, a request for 1..7 misses there (stop at the first miss), recomputes 3..6,
    caches its new [1..4] and leaves [1..6] to the block that already holds it."""
    m = BM.PrefixCachingModel(8, 2)
    assert m.add_seq_tokens("P", [1, 2, 3]) == (BM.OK, 0)
    assert m.fork("P", "Q") == BM.OK
    m.append_token("Q", 4)  # Q copies the shared tail on write and caches [1..4]
    m.append_token("P", 4)
    for t in (5, 6):        # P first: P caches [1..6]
        m.append_token("P", t)
        m.append_token("Q", t)
    x, p1, p2 = m.tables["P"]
    _, q1, q2 = m.tables["Q"]
    assert m.index[(1, 2, 3, 4)] == q1 and m.index[(1, 2, 3, 4, 5, 6)] == p2
    m.free_seq("Q")   # q2 uncached -> free; q1 -> idle
    m.free_seq("P")   # p2 -> idle, p1 -> free, x -> idle
    assert m.idle == [q1, p2, x] and len(m.free) == 5
    assert m.add_seq("F", 12) == BM.OK and m.evictions == 1  # 6 blocks: 5 free + q1 evicted
    assert (1, 2, 3, 4) not in m.index and m.index[(1, 2, 3, 4, 5, 6)] == p2
    m.free_seq("F")   # F's blocks were never cached: back to the free list
    st, hit = m.add_seq_tokens("R", [1, 2, 3, 4, 5, 6, 7])
    assert st == BM.OK and hit == 2 and m.tables["R"][0] == x
    assert m.index[(1, 2, 3, 4)] == m.tables["R"][1]
    assert m.index[(1, 2, 3, 4, 5, 6)] == p2 and m.tables["R"][2] not in m.entry
    _check(m)


@pytest.mark.parametrize("seed", range(30))
def test_random_traces_hit_exactly_the_cached_prefixes(seed):
    """Random requests over a small vocabulary (so prefixes repeat), forks, appends with and without token ids,
    releases and pressure.  Every lookup equals brute force over the cached prefixes, and every reused block
    stands for exactly the request's tokens."""
    rng = random.Random(seed)
    B = rng.choice([2, 4, 8])
    m = BM.PrefixCachingModel(rng.randint(24, 64), B, rng.sample(range(64), 64)[:0] or None)
    prompts = [[rng.randrange(3) for _ in range(rng.randint(1, 6 * B))] for _ in range(6)]
    live, nid = [], 0
    for _ in range(120):
        op = rng.random()
        if op < 0.35:
            base = rng.choice(prompts)
            toks = base[:rng.randint(1, len(base))] + [rng.randrange(3) for _ in range(rng.randint(0, B))]
            cached = {tuple(m.cached_prefix(b)) for b in m.entry}
            expect = 0
            while (expect + 1) * B <= len(toks) and tuple(toks[:(expect + 1) * B]) in cached:
                expect += 1
            st, hit = m.add_seq_tokens(nid, toks)
            if st == BM.OK:
                assert hit == expect * B
                for i, b in enumerate(m.tables[nid][:expect]):
                    assert m.cached_prefix(b) == toks[:(i + 1) * B]
                live.append(nid)
            else:
                assert st == BM.ERR_NO_FREE_BLOCKS
            nid += 1
        elif op < 0.5 and live:
            p = rng.choice(live)
            assert m.fork(p, nid) == BM.OK
            live.append(nid)
            nid += 1
        elif op < 0.8 and live:
            seqs = rng.sample(live, rng.randint(1, len(live)))
            toks = None if rng.random() < 0.2 else [rng.randrange(3) for _ in seqs]
            st, slots, pairs, _ = m.append_tokens(seqs, toks)
            assert st in (BM.OK, BM.ERR_NO_FREE_BLOCKS)
        elif live:
            s = rng.choice(live)
            live.remove(s)
            assert m.free_seq(s) == BM.OK
        _check(m)

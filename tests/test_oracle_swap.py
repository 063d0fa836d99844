"""Pins for swapping in the block manager model ([P1] section 19: preemption by swapping -- physical blocks move to
host memory and come back when device blocks are released).

Every test runs a payload model beside the managers: device and host pools of token ids, written by appends, copied
by the copy-on-write pairs and by the swap pairs.  Whatever the manager does, every sequence must keep reading its
own token history through its table, wherever its blocks are.
"""

import random

import pytest

from oracle import block_manager as BM


class Payload:
    def __init__(self, m):
        self.m = m
        self.dev = [[None] * m.block_size for _ in range(m.num_blocks)]
        self.host = [[None] * m.block_size for _ in range(max(len(m.host_ref), 1))]
        self.hist = {}

    def add(self, seq, n, start_token):
        """Fill a new sequence's n tokens (its prefill) with ids start_token .. start_token + n - 1."""
        B = self.m.block_size
        self.hist[seq] = list(range(start_token, start_token + n))
        for t, tok in enumerate(self.hist[seq]):
            self.dev[self.m.tables[seq][t // B]][t % B] = tok

    def append(self, seq, slot, pair, tok):
        B = self.m.block_size
        if pair is not None:
            self.dev[pair[1]] = list(self.dev[pair[0]])
        self.dev[slot // B][slot % B] = tok
        self.hist[seq].append(tok)

    def fork(self, parent, child):
        self.hist[child] = list(self.hist[parent])

    def swap_out(self, pairs):
        for b, hb in pairs:
            self.host[hb] = list(self.dev[b])

    def swap_in(self, pairs):
        for hb, b in pairs:
            self.dev[b] = list(self.host[hb])

    def check(self):
        m, B = self.m, self.m.block_size
        for seq, hist in self.hist.items():
            pool = self.host if seq in m.swapped else self.dev
            seen = [pool[m.tables[seq][t // B]][t % B] for t in range(m.lens[seq])]
            assert seen == hist, f"sequence {seq} reads {seen}, wrote {hist}"
        # references: device counts come from resident tables, host counts from swapped ones
        dev = [0] * m.num_blocks
        host = [0] * len(m.host_ref)
        for seq, t in m.tables.items():
            for b in t:
                (host if seq in m.swapped else dev)[b] += 1
        assert dev == m.ref and host == m.host_ref
        assert sorted(m.host_free) == [h for h in range(len(host)) if host[h] == 0]


def test_swap_out_frees_device_blocks_and_swap_in_restores_the_history():
    """[P1] section 19: the pool is full, a running sequence is swapped out, its device blocks serve another
    request, and when they are released it comes back with its cache intact."""
    m = BM.BlockManagerModel(6, 4)
    assert m.enable_host_pool(8) == BM.OK
    pl = Payload(m)
    assert m.add_seq("A", 10) == BM.OK  # 3 blocks
    pl.add("A", 10, 100)
    assert m.add_seq("B", 12) == BM.OK  # 3 blocks: pool full
    pl.add("B", 12, 200)
    assert m.add_seq("C", 4) == BM.ERR_NO_FREE_BLOCKS
    a_blocks = list(m.tables["A"])
    st, pairs = m.swap_out(["A"])
    assert st == BM.OK and [b for b, _ in pairs] == a_blocks and len(m.free) == 3
    pl.swap_out(pairs)
    pl.check()
    # a swapped sequence is off the device: no appends, forks or batches
    assert m.append_slot("A")[0] == BM.ERR_INVALID_ARG
    assert m.fork("A", "A2") == BM.ERR_INVALID_ARG
    assert m.build_batch(["A"], 4)[0] == BM.ERR_INVALID_ARG
    assert m.add_seq("C", 9) == BM.OK  # reuses A's released device blocks
    pl.add("C", 9, 300)
    assert sorted(m.tables["C"]) == sorted(a_blocks)
    assert m.swap_in(["A"])[0] == BM.ERR_NO_FREE_BLOCKS  # not until device blocks are released
    assert m.free_seq("C") == BM.OK
    del pl.hist["C"]
    st, pairs = m.swap_in(["A"])
    assert st == BM.OK and len(pairs) == 3 and m.swap_stats()["host_free"] == 8
    pl.swap_in(pairs)
    pl.check()
    st, slot, src, dst = m.append_slot("A")
    assert st == BM.OK and src == -1
    pl.append("A", slot, None, 110)
    pl.check()


def test_a_fork_family_swapped_together_keeps_its_sharing():
    m = BM.BlockManagerModel(32, 4)
    m.enable_host_pool(32)
    pl = Payload(m)
    m.add_seq(0, 10)
    pl.add(0, 10, 0)
    for c in (1, 2, 3):
        m.fork(0, c)
        pl.fork(0, c)
    for s in (0, 1, 2, 3):  # copy-on-write of the shared tail, one new token each
        st, slot, src, dst = m.append_slot(s)
        pl.append(s, slot, (src, dst) if src >= 0 else None, 50 + s)
    st, pairs = m.swap_out([0, 1, 2, 3])
    assert st == BM.OK and len(pairs) == 2 + 4  # 2 shared full blocks once, 4 private tails
    shared_host = [hb for b, hb in pairs[:2]]
    assert [m.host_ref[h] for h in shared_host] == [4, 4]
    pl.swap_out(pairs)
    pl.check()
    st, pairs = m.swap_in([0, 1, 2, 3])
    assert st == BM.OK
    pl.swap_in(pairs)
    assert [m.ref[b] for b in m.tables[0][:2]] == [4, 4]  # shared again
    assert all(m.tables[s][:2] == m.tables[0][:2] for s in (1, 2, 3))
    pl.check()


def test_swapping_part_of_a_family_copies_the_shared_blocks():
    """A block also used outside the swapped list keeps those references on the device; the host copy belongs to
    the swapped sequences, which get private blocks when they come back."""
    m = BM.BlockManagerModel(32, 4)
    m.enable_host_pool(32)
    pl = Payload(m)
    m.add_seq(0, 8)
    pl.add(0, 8, 0)
    m.fork(0, 1)
    pl.fork(0, 1)
    shared = list(m.tables[0])
    st, pairs = m.swap_out([1])
    assert st == BM.OK and [b for b, _ in pairs] == shared
    assert [m.ref[b] for b in shared] == [1, 1]  # 0 keeps them
    pl.swap_out(pairs)
    st, pairs = m.swap_in([1])
    pl.swap_in(pairs)
    assert not set(m.tables[1]) & set(shared)
    pl.check()


def test_swaps_are_all_or_nothing():
    m = BM.BlockManagerModel(8, 4)
    m.enable_host_pool(2)
    m.add_seq(0, 12)  # 3 blocks
    before = (list(m.free), list(m.ref), list(m.host_free), dict(m.tables))
    assert m.swap_out([0])[0] == BM.ERR_NO_FREE_BLOCKS  # 3 host blocks needed, 2 there
    assert m.swap_out([0, 0])[0] == BM.ERR_INVALID_ARG
    assert m.swap_out([7])[0] == BM.ERR_NOT_FOUND
    assert m.swap_in([0])[0] == BM.ERR_INVALID_ARG  # not swapped
    assert (list(m.free), list(m.ref), list(m.host_free), dict(m.tables)) == before
    # freeing a swapped sequence returns its host blocks
    m2 = BM.BlockManagerModel(8, 4)
    m2.enable_host_pool(4)
    m2.add_seq(0, 5)
    assert m2.swap_out([0])[0] == BM.OK and m2.swap_stats()["host_free"] == 2
    assert m2.free_seq(0) == BM.OK and m2.swap_stats() == {"num_swapped": 0, "host_free": 4, "host_blocks": 4}
    assert m2.enable_host_pool(4) == BM.ERR_INVALID_ARG  # once


def test_swap_with_the_prefix_cache():
    """A cached block released by a swap-out stays cached (idle) on the device; the swapped sequence comes back
    into fresh blocks and its chain goes on: its next full block is cached."""
    m = BM.PrefixCachingModel(16, 2)
    m.enable_host_pool(16)
    assert m.add_seq_tokens("A", [1, 2, 3, 4, 5]) == (BM.OK, 0)
    st, pairs = m.swap_out(["A"])
    assert st == BM.OK and m.stats()["num_idle"] == 2
    assert m.add_seq_tokens("B", [1, 2, 3, 4, 9]) == (BM.OK, 4)  # the idle cached blocks serve B
    st, pairs = m.swap_in(["A"])
    assert st == BM.OK
    m.append_token("A", 6)  # [5, 6] completes A's third block
    assert (1, 2, 3, 4, 5, 6) in m.index
    assert m.append_tokens(["A"], [7])[0] == BM.OK
    assert m.swap_out(["A"])[0] == BM.OK and m.append_tokens(["A"], [8])[0] == BM.ERR_INVALID_ARG


@pytest.mark.parametrize("seed", range(30))
def test_random_traces_keep_every_history(seed):
    rng = random.Random(seed)
    B = rng.choice([2, 4, 8])
    cached = seed % 2 == 1
    nb, nh = rng.randint(12, 40), rng.randint(8, 40)
    m = BM.PrefixCachingModel(nb, B) if cached else BM.BlockManagerModel(nb, B)
    m.enable_host_pool(nh)
    pl = Payload(m)
    live, nid, tok = [], 0, 1000
    for _ in range(150):
        op = rng.random()
        resident = [s for s in live if s not in m.swapped]
        swapped = [s for s in live if s in m.swapped]
        if op < 0.2:
            n = rng.randint(1, 4 * B)
            if m.add_seq(nid, n) == BM.OK:
                pl.add(nid, n, tok)
                tok += n
                live.append(nid)
            nid += 1
        elif op < 0.3 and resident:
            p = rng.choice(resident)
            assert m.fork(p, nid) == BM.OK
            pl.fork(p, nid)
            live.append(nid)
            nid += 1
        elif op < 0.55 and resident:
            s = rng.choice(resident)
            st, slot, src, dst = m.append_slot(s)
            if st == BM.OK:
                pl.append(s, slot, (src, dst) if src >= 0 else None, tok)
                tok += 1
        elif op < 0.7 and resident:
            group = rng.sample(resident, rng.randint(1, min(3, len(resident))))
            st, pairs = m.swap_out(group)
            if st == BM.OK:
                pl.swap_out(pairs)
        elif op < 0.85 and swapped:
            group = rng.sample(swapped, rng.randint(1, min(3, len(swapped))))
            st, pairs = m.swap_in(group)
            if st == BM.OK:
                pl.swap_in(pairs)
        elif live:
            s = rng.choice(live)
            live.remove(s)
            assert m.free_seq(s) == BM.OK
            del pl.hist[s]
        pl.check()

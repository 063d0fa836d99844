"""Pins for oracle/block_manager.py: the pages' traces, the teaching tests, and invariants."""

import random

import numpy as np

from conftest import golden
from oracle import attention as A
from oracle import block_manager as BM


def _refs(m, blocks):
    return {str(b): m.ref[b] for b in blocks}


def test_fork_35_trace():
    g = golden("block_manager_traces.json")["fork_35"]
    B, nb = g["block_size"], g["num_blocks"]
    prefix = g["pop_order_prefix"]
    order = prefix + [b for b in range(nb) if b not in prefix]
    m = BM.BlockManagerModel(nb, B, order)
    A_, B_ = 1, 2
    assert m.add_seq(A_, g["prompt"]) == BM.OK
    assert m.tables[A_] == g["after_setup"]["A"]
    assert _refs(m, [10, 11, 12]) == g["after_setup"]["refs"]
    assert m.fork(A_, B_) == BM.OK
    assert m.tables[B_] == g["after_fork"]["B"]
    assert _refs(m, [10, 11, 12]) == g["after_fork"]["refs"]
    st, slot, src, dst = m.append_slot(A_)
    assert st == BM.OK and divmod(slot, B) == (g["append_A"]["slot_block"], g["append_A"]["slot_offset"])
    assert [src, dst] == g["append_A"]["cow"]
    st, slot, src, dst = m.append_slot(B_)
    assert st == BM.OK and divmod(slot, B) == (g["append_B"]["slot_block"], g["append_B"]["slot_offset"])
    assert src == -1 and dst == -1
    e = g["after_step"]
    assert m.tables[A_] == e["A"] and m.tables[B_] == e["B"]
    assert _refs(m, [10, 11, 12, 13]) == e["refs"]
    s = m.stats()
    assert s["num_used"] == e["blocks_in_use"] and s["num_used"] * B == e["slots"]
    assert s["stored_tokens"] == e["stored_tokens"] and s["tail_waste_slots"] == e["tail_waste"]
    unshared = sum(-(-m.lens[x] // B) for x in (A_, B_))
    assert unshared == e["unshared_blocks"] and (unshared - s["num_used"]) * B == e["saved_slots"]
    assert m.free_seq(A_) == BM.OK
    f = g["after_free_A"]
    assert m.tables[B_] == f["B"] and _refs(m, [10, 11, 12, 13]) == f["refs"]
    assert m.pop_order()[0] == f["freed"][0]  # the released block is handed out next (LIFO)


def test_exercise_2_trace():
    g = golden("block_manager_traces.json")["exercise_2"]
    B = g["block_size"]
    m = BM.BlockManagerModel(g["num_blocks"], B)
    assert m.add_seq("A", g["prompt"]) == BM.OK
    assert len(m.tables["A"]) == g["initial_blocks"]
    assert m.fork("A", "B") == BM.OK
    assert _refs(m, [0, 1, 2]) == g["after_fork_refs"]
    events = {e["token"]: e for e in g["events"]}
    for tok in range(g["prompt"], g["prompt"] + g["appends_A"]):
        fresh_before = len(m.tables["A"])
        st, slot, src, dst = m.append_slot("A")
        assert st == BM.OK
        if tok in events:
            e = events[tok]
            assert divmod(slot, B) == (e["block"], e["offset"])
            assert ([src, dst] if src >= 0 else None) == e["cow"]
            assert (len(m.tables["A"]) > fresh_before) == e.get("fresh", False)
    f = g["final"]
    assert m.tables["A"] == f["A"] and m.tables["B"] == f["B"]
    assert m.lens["A"] == f["len_A"] and m.lens["B"] == f["len_B"]
    assert _refs(m, range(5)) == f["refs"]
    s = m.stats()
    assert s["num_used"] == f["blocks_in_use"] and s["num_used"] * B == f["slots"]
    assert s["stored_tokens"] == f["stored_tokens"] and s["tail_waste_slots"] == f["tail_waste"]


def test_teaching_t1_capacity():
    t = golden("block_manager_traces.json")["teaching_tests"]["t1"]
    m = BM.BlockManagerModel(t["num_blocks"], t["block_size"])
    for i, L in enumerate(t["lengths"]):
        assert m.add_seq(i, L) == BM.OK
    slots = sum(len(m.tables[i]) for i in range(4)) * t["block_size"]
    assert slots == t["slots"] and slots - sum(t["lengths"]) == t["waste"]
    assert m.stats()["num_free"] == 0


def _payload_pool(nb, B):
    return np.zeros((nb, 1, B, 1)), np.zeros((nb, 1, B, 1))


def test_teaching_t2_cow_isolation_and_t5_release():
    t = golden("block_manager_traces.json")["teaching_tests"]
    t2 = t["t2"]
    B = t2["block_size"]
    m = BM.BlockManagerModel(t2["num_blocks"], B)
    kp, vp = _payload_pool(t2["num_blocks"], B)
    prompt = [(float(i), float(i * 10)) for i in range(t2["prompt_len"])]
    assert m.add_seq("A", len(prompt)) == BM.OK
    slots = [A.translate(i, B, m.tables["A"])[3] for i in range(len(prompt))]
    A.append_kv(kp, vp, np.array([[[k]] for k, _ in prompt]), np.array([[[v]] for _, v in prompt]), slots)
    assert m.fork("A", "B") == BM.OK
    for seq, (k, v) in (("A", t2["payload_A"]), ("B", t2["payload_B"])):
        st, slot, src, dst = m.append_slot(seq)
        assert st == BM.OK
        if src >= 0:
            A.copy_blocks(kp, vp, [(src, dst)])  # copy first, then write the new token
        A.append_kv(kp, vp, np.array([[[k]]]), np.array([[[v]]]), [slot])
    tail_A, tail_B = m.tables["A"][1], m.tables["B"][1]
    assert tail_A != tail_B
    assert (kp[tail_A, 0, 2, 0], vp[tail_A, 0, 2, 0]) == tuple(t2["payload_A"])
    assert (kp[tail_B, 0, 2, 0], vp[tail_B, 0, 2, 0]) == tuple(t2["payload_B"])
    assert (kp[tail_A, 0, 0, 0], vp[tail_A, 0, 0, 0]) == prompt[t2["tail_A_slot0_is_prompt_index"]]
    # T5: releasing every sequence returns the whole pool
    assert m.free_seq("A") == BM.OK and m.free_seq("B") == BM.OK
    assert len(m.free) == t2["num_blocks"] and all(r == 0 for r in m.ref)


def test_teaching_t4_exhaustion_is_transactional():
    t4 = golden("block_manager_traces.json")["teaching_tests"]["t4"]
    m = BM.BlockManagerModel(t4["num_blocks"], t4["block_size"])
    assert m.add_seq("s", t4["prompt_len"]) == BM.OK
    before = (list(m.tables["s"]), m.lens["s"], list(m.free), list(m.ref))
    assert m.append_slot("s")[0] == BM.ERR_NO_FREE_BLOCKS
    assert (list(m.tables["s"]), m.lens["s"], list(m.free), list(m.ref)) == before
    assert m.add_seq("t", 1) == BM.ERR_NO_FREE_BLOCKS and "t" not in m.tables


def test_errors_change_nothing():
    m = BM.BlockManagerModel(4, 4)
    assert m.add_seq(1, 0) == BM.ERR_INVALID_ARG
    assert m.add_seq(1, 5) == BM.OK
    assert m.add_seq(1, 1) == BM.ERR_EXISTS
    assert m.fork(9, 2) == BM.ERR_NOT_FOUND
    assert m.fork(1, 1) == BM.ERR_EXISTS
    assert m.append_slot(9)[0] == BM.ERR_NOT_FOUND
    assert m.free_seq(9) == BM.ERR_NOT_FOUND
    assert m.tables == {1: [0, 1]} and m.ref == [1, 1, 0, 0]


def _check_invariants(m):
    total_refs = sum(m.ref)
    assert total_refs == sum(len(t) for t in m.tables.values())
    used = {b for t in m.tables.values() for b in t}
    assert used.isdisjoint(m.free)
    assert used | set(m.free) == set(range(m.num_blocks))
    assert len(m.free) == len(set(m.free))
    for b in range(m.num_blocks):
        assert (m.ref[b] > 0) == (b in used)
    for s, t in m.tables.items():
        assert len(t) == -(-m.lens[s] // m.block_size)
        st = m.stats()
        assert 0 <= st["tail_waste_slots"]


def test_random_operations_keep_invariants_and_write_only_private_blocks():
    rng = random.Random(11)
    for trial in range(30):
        nb, B = rng.choice([(8, 4), (32, 8), (64, 16)])
        m = BM.BlockManagerModel(nb, B, rng.sample(range(nb), nb))
        next_id = 0
        for _ in range(200):
            op = rng.random()
            live = list(m.tables)
            if op < 0.25 or not live:
                m.add_seq(next_id, rng.randint(1, 3 * B))
                next_id += 1
            elif op < 0.4:
                m.fork(rng.choice(live), next_id)
                next_id += 1
            elif op < 0.85:
                seq = rng.choice(live)
                st, slot, src, dst = m.append_slot(seq)
                if st == BM.OK:
                    assert m.ref[slot // B] == 1  # a written block is never shared
                    assert slot // B == m.tables[seq][-1]
                    if src >= 0:
                        assert m.ref[dst] == 1 and m.ref[src] >= 1
            elif op < 0.95:
                seqs = rng.sample(live, rng.randint(1, len(live)))
                before = (dict((k, list(v)) for k, v in m.tables.items()), dict(m.lens), list(m.free), list(m.ref))
                st, slots, pairs, failed = m.append_slots(seqs)
                if st != BM.OK:
                    after = (dict((k, list(v)) for k, v in m.tables.items()), dict(m.lens), list(m.free), list(m.ref))
                    assert after == before
                else:
                    assert len(set(slots)) == len(slots)
                    assert len({d for _, d in pairs}) == len(pairs)
                    assert not ({d for _, d in pairs} & {s for s, _ in pairs})
            else:
                m.free_seq(rng.choice(live))
            _check_invariants(m)


def test_random_operations_keep_the_models_own_invariants_with_prefix_caching():
    """The oracle's check_invariants (counts equal table entries, free and idle blocks unreferenced and listed once,
    ceil(S / B) blocks per sequence) holds after every operation, with and without the prefix cache; a pin of the
    plan-then-commit form of fork / append_slot / free_seq against the same random sequences as above."""
    rng = random.Random(23)
    for trial in range(20):
        nb, B = rng.choice([(8, 4), (32, 8), (64, 16)])
        caching = trial % 2 == 1
        m = (BM.PrefixCachingModel if caching else BM.BlockManagerModel)(nb, B, rng.sample(range(nb), nb))
        next_id = 0
        prompts = [[rng.randrange(50) for _ in range(3 * B)] for _ in range(3)]
        for _ in range(150):
            live = [s for s in m.tables if s not in m.swapped]
            op = rng.random()
            if op < 0.25 or not live:
                if caching:
                    p = rng.choice(prompts)
                    m.add_seq_tokens(next_id, p[:rng.randint(1, len(p))])
                else:
                    m.add_seq(next_id, rng.randint(1, 3 * B))
                next_id += 1
            elif op < 0.4:
                m.fork(rng.choice(live), next_id)
                next_id += 1
            elif op < 0.85:
                seq = rng.choice(live)
                st, slot, src, dst = m.append_slot(seq)
                if st == BM.OK:
                    assert m.ref[slot // B] == 1 and slot // B == m.tables[seq][-1]
            else:
                m.free_seq(rng.choice(live))
            m.check_invariants()

"""Pure-Python model of the host block manager.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  The C++ block manager
in the product library is checked against this model, operation by operation,
on seeded random operation sequences.

Rules, as the pages state them:
  * A sequence of S tokens holds ceil(S / B) blocks ([P1] section 8 item 3).
  * Fork copies the parent's block table and raises the reference count of
    every block in it; no data moves ([P1] section 16 step 2).
  * Appending at position S ([P1] sections 15-16):
      - S mod B == 0: the tail is full, take a fresh block and write offset 0;
      - S mod B != 0 and the tail block is shared (ref > 1): copy-on-write --
        take a fresh block, copy the tail's valid tokens into it, drop the old
        block's count by one, point the table at the new block (ref 1), write
        there;
      - S mod B != 0 and the tail is private (ref == 1): write in place.
  * On release every block's count drops by one; a block reaching 0 returns
    to the free list ([P1] section 17).
  * Running out of free blocks fails the operation and changes nothing
    ([P1] section 20, test 4: exhaustion leaves the sequence untouched).

Readings taken where the pages leave a detail open:
  * The free list is a LIFO stack: the most recently released block is handed
    out first.  [P1]'s teaching model pops from the end of a list that starts
    as the block ids in reverse order, so with no explicit order blocks
    0, 1, 2, ... are handed out in that order.  ``pop_order`` lets a caller
    fix the initial hand-out order (the first entry is handed out first).
  * The copy-on-write copy is reported as a (src, dst) pair; the device copy
    clones the whole block.
  * A batch append is all-or-nothing: when one sequence of the batch cannot
    get a block, the appends already done in that batch are undone in reverse
    order, which restores the free list exactly.
  * Operations on unknown or duplicate sequence ids fail with NOT_FOUND or
    EXISTS and change nothing.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

OK = 0
ERR_INVALID_ARG = 1
ERR_NO_FREE_BLOCKS = 3
ERR_EXISTS = 4
ERR_NOT_FOUND = 5


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int,
                 pop_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        if pop_order is None:
            pop_order = range(num_blocks)
        pop_order = [int(b) for b in pop_order]
        if sorted(pop_order) != list(range(num_blocks)):
            raise ValueError("pop_order must be a permutation of the block ids")
        # top of the stack is the end of the list
        self.free: List[int] = list(reversed(pop_order))
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.cow_copies = 0
        # swapping ([P1] section 19): a host pool of blocks, and the sequences whose tables hold host ids
        self.host_free: List[int] = []
        self.host_ref: List[int] = []
        self.swapped: set = set()

    # -- allocation -------------------------------------------------------
    def _available(self) -> int:
        """Blocks an allocation may take."""
        return len(self.free)

    def _pop(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def add_seq(self, seq: int, num_tokens: int) -> int:
        if num_tokens <= 0:
            return ERR_INVALID_ARG
        if seq in self.tables:
            return ERR_EXISTS
        need = -(-num_tokens // self.block_size)
        if self._available() < need:
            return ERR_NO_FREE_BLOCKS
        self.tables[seq] = [self._pop() for _ in range(need)]
        self.lens[seq] = num_tokens
        return OK

    # -- the sharing rules of [P1] sections 14-17 --------------------------------
    # Each operation checks its preconditions first and changes nothing when one
    # fails; then it applies its whole effect.  Two primitives carry the
    # reference counting of section 17: _pop (a free block becomes referenced
    # once) and _unref (one reference goes away; at zero the block is released).

    def _unref(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self._release(b)

    def fork(self, parent: int, child: int) -> int:
        """The child becomes a second owner of every block of the parent ([P1] sections 14 and 16).

        Pre: parent known and resident; child new.
        Post: the child's table and length equal the parent's; each of those
        blocks has one reference more; the free set is unchanged (no data moves).
        """
        if parent not in self.tables:
            return ERR_NOT_FOUND
        if child in self.tables:
            return ERR_EXISTS
        if parent in self.swapped:
            return ERR_INVALID_ARG
        shared = self.tables[parent]
        self.tables[child] = list(shared)
        self.lens[child] = self.lens[parent]
        for b in shared:
            self.ref[b] += 1
        return OK

    def _placement(self, seq: int) -> str:
        """Where position S = len(seq) goes ([P1] sections 15-16):

        'open'   S is a multiple of B: the tail is full (or there is none), so
                 a fresh block is added to the table;
        'clone'  the tail is partly filled and shared (ref > 1): a shared block
                 is immutable (section 15), so the sequence takes a private copy
                 of it -- a fresh block, with (tail, fresh) reported for the
                 device copy;
        'write'  the tail is partly filled and only this sequence holds it: the
                 token goes there.
        """
        if self.lens[seq] % self.block_size == 0:
            return "open"
        return "clone" if self.ref[self.tables[seq][-1]] > 1 else "write"

    def append_slot(self, seq: int) -> Tuple[int, int, int, int]:
        """Reserve the slot of position S = len(seq).  Returns (status, slot, copy src, copy dst).

        Pre: seq known and resident; 'open' and 'clone' need a block to take
        (else NO_FREE_BLOCKS, nothing changed).
        Post: len(seq) = S + 1; the table covers ceil((S + 1) / B) blocks and
        its last block is held by this sequence alone; the slot is
        table[S // B] * B + S % B ([P1] section 7).  A clone moves this
        sequence's reference from the shared tail to its copy; the other owners
        keep the tail unchanged.
        """
        if seq not in self.tables:
            return ERR_NOT_FOUND, -1, -1, -1
        if seq in self.swapped:
            return ERR_INVALID_ARG, -1, -1, -1
        where = self._placement(seq)
        if where != "write" and self._available() == 0:
            return ERR_NO_FREE_BLOCKS, -1, -1, -1
        table, S = self.tables[seq], self.lens[seq]
        src = dst = -1
        if where == "open":
            table.append(self._pop())
        elif where == "clone":
            src, dst = table[-1], self._pop()
            table[-1] = dst
            self._unref(src)  # still held by the other owners: never released here
            self.cow_copies += 1
        self.lens[seq] = S + 1
        return OK, table[S // self.block_size] * self.block_size + S % self.block_size, src, dst

    def _undo_append(self, seq: int, src: int, dst: int) -> None:
        """The inverse of one append_slot (a failed batch is rolled back newest first, which restores
        the free list exactly: every block goes back on top of the stack it came from)."""
        table = self.tables[seq]
        self.lens[seq] -= 1
        if src >= 0:  # drop the copy; the sequence shares the old tail again
            table[-1] = src
            self.ref[src] += 1
            self.ref[dst] = 0
            self.free.append(dst)
            self.cow_copies -= 1
        elif self.lens[seq] % self.block_size == 0:  # give back the block the append opened
            b = table.pop()
            self.ref[b] = 0
            self.free.append(b)

    def append_slots(self, seqs: Sequence[int]) -> Tuple[int, List[int], List[Tuple[int, int]], int]:
        """Batch append, all-or-nothing.  Returns (status, slots, cow_pairs, failed_index)."""
        done: List[Tuple[int, int, int]] = []
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for i, seq in enumerate(seqs):
            st, slot, src, dst = self.append_slot(seq)
            if st != OK:
                for s, a, b in reversed(done):
                    self._undo_append(s, a, b)
                return st, [], [], i
            done.append((seq, src, dst))
            slots.append(slot)
            if src >= 0:
                pairs.append((src, dst))
        return OK, slots, pairs, -1

    def free_seq(self, seq: int) -> int:
        """A finished sequence gives up its reference to each of its blocks ([P1] section 17).

        Pre: seq known.  Post: seq is gone; each of its blocks has one
        reference fewer, and those no one holds any more are free again, in
        table order (reading: the last block released is the first reused).
        """
        if seq not in self.tables:
            return ERR_NOT_FOUND
        if seq in self.swapped:
            self._free_host(seq)
            return OK
        for b in self.tables.pop(seq):
            self._unref(b)
        del self.lens[seq]
        return OK

    def check_invariants(self) -> None:
        """The bookkeeping facts of [P1] sections 8 and 17, asserted on the whole state:
        every resident sequence of S tokens holds ceil(S / B) blocks; a block's count is the number of
        table entries naming it; free blocks are referenced by no one and appear once."""
        count = [0] * self.num_blocks
        for seq, table in self.tables.items():
            if seq in self.swapped:
                continue
            assert len(table) == -(-self.lens[seq] // self.block_size), seq
            for b in table:
                count[b] += 1
        assert count == self.ref, "reference counts differ from the tables"
        free = list(self.free) + list(getattr(self, "idle", []))
        assert len(set(free)) == len(free), "a block is free twice"
        assert all(self.ref[b] == 0 for b in free), "a referenced block is free"

    def _free_host(self, seq: int) -> None:
        for hb in self.tables[seq]:
            self.host_ref[hb] -= 1
            if self.host_ref[hb] == 0:
                self.host_free.append(hb)
        self.swapped.discard(seq)
        del self.tables[seq]
        del self.lens[seq]

    # -- swapping ([P1] section 19, "Preemption via Swapping") ---------------
    def enable_host_pool(self, num_host_blocks: int, pop_order: Optional[Sequence[int]] = None) -> int:
        """A pool of host blocks for swapped-out sequences (host ids 0 .. num_host_blocks - 1)."""
        if num_host_blocks <= 0 or self.host_ref:
            return ERR_INVALID_ARG
        order = list(range(num_host_blocks)) if pop_order is None else [int(b) for b in pop_order]
        if sorted(order) != list(range(num_host_blocks)):
            return ERR_INVALID_ARG
        self.host_free = list(reversed(order))
        self.host_ref = [0] * num_host_blocks
        return OK

    def _release(self, b: int) -> None:
        """A device block whose last reference went away."""
        self.free.append(b)

    def _distinct_blocks(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        """(block, references from `seqs`) in order of first appearance (sequence order, then table order)."""
        count: Dict[int, int] = {}
        order: List[int] = []
        for seq in seqs:
            for b in self.tables[seq]:
                if b not in count:
                    count[b] = 0
                    order.append(b)
                count[b] += 1
        return [(b, count[b]) for b in order]

    def _swap_check(self, seqs: Sequence[int], want_swapped: bool) -> int:
        if len(set(seqs)) != len(seqs):
            return ERR_INVALID_ARG
        for seq in seqs:
            if seq not in self.tables:
                return ERR_NOT_FOUND
            if (seq in self.swapped) != want_swapped:
                return ERR_INVALID_ARG
        return OK

    def swap_out(self, seqs: Sequence[int]) -> Tuple[int, List[Tuple[int, int]]]:
        """Move these resident sequences to host blocks, all-or-nothing.  Returns (status, [(device block, host
        block)]) -- the copies to make before the released device blocks are reused.

        Each distinct device block the sequences reference gets one host block, which takes over their
        references; a block also used by a sequence outside the list keeps its other references (its host
        copy belongs to the listed sequences only), any other block is released.
        """
        st = self._swap_check(seqs, False)
        if st != OK:
            return st, []
        blocks = self._distinct_blocks(seqs)
        if len(self.host_free) < len(blocks):
            return ERR_NO_FREE_BLOCKS, []
        pairs, where = [], {}
        for b, c in blocks:
            hb = self.host_free.pop()
            self.host_ref[hb] = c
            self.ref[b] -= c
            if self.ref[b] == 0:
                self._release(b)
            pairs.append((b, hb))
            where[b] = hb
        for seq in seqs:
            self.tables[seq] = [where[b] for b in self.tables[seq]]
            self.swapped.add(seq)
        return OK, pairs

    def swap_in(self, seqs: Sequence[int]) -> Tuple[int, List[Tuple[int, int]]]:
        """Bring these swapped sequences back into fresh device blocks, all-or-nothing.  Returns (status,
        [(host block, device block)]) -- the copies to make before the sequences are decoded."""
        st = self._swap_check(seqs, True)
        if st != OK:
            return st, []
        blocks = self._distinct_blocks(seqs)
        if self._available() < len(blocks):
            return ERR_NO_FREE_BLOCKS, []
        pairs, where = [], {}
        for hb, c in blocks:
            b = self._pop()
            self.ref[b] = c
            self.host_ref[hb] -= c
            if self.host_ref[hb] == 0:
                self.host_free.append(hb)
            pairs.append((hb, b))
            where[hb] = b
        for seq in seqs:
            self.tables[seq] = [where[hb] for hb in self.tables[seq]]
            self.swapped.discard(seq)
        return OK, pairs

    # -- queries ----------------------------------------------------------
    def build_batch(self, seqs: Sequence[int], max_blocks: int) -> Tuple[int, List[List[int]], List[int]]:
        tables, lens = [], []
        for seq in seqs:
            if seq not in self.tables:
                return ERR_NOT_FOUND, [], []
            if seq in self.swapped:
                return ERR_INVALID_ARG, [], []
            t = self.tables[seq]
            if len(t) > max_blocks:
                return ERR_INVALID_ARG, [], []
            tables.append(t + [0] * (max_blocks - len(t)))
            lens.append(self.lens[seq])
        return OK, tables, lens

    def pop_order(self) -> List[int]:
        """The free list in hand-out order (next block first)."""
        return list(reversed(self.free))

    def stats(self) -> Dict[str, int]:
        """Pool accounting in the terms of [P1] section 17.

        A block's fill is the number of valid tokens it holds (the largest
        count over the sequences that reference it); stored tokens sum the
        fills, so shared blocks count once, and tail waste is the slots of
        blocks in use minus the stored tokens.
        """
        fill: Dict[int, int] = {}
        for seq, table in self.tables.items():
            if seq in self.swapped:  # host blocks: not part of the device pool
                continue
            length = self.lens[seq]
            for lb, b in enumerate(table):
                valid = min(self.block_size, length - lb * self.block_size)
                fill[b] = max(fill.get(b, 0), valid)
        used = sum(1 for r in self.ref if r > 0)
        stored = sum(fill.values())
        return {
            "num_blocks": self.num_blocks,
            "num_free": len(self.free),
            "num_used": used,
            "num_seqs": len(self.tables),
            "cow_copies": self.cow_copies,
            "stored_tokens": stored,
            "tail_waste_slots": used * self.block_size - stored,
        }

    def swap_stats(self) -> Dict[str, int]:
        return {"num_swapped": len(self.swapped), "host_free": len(self.host_free),
                "host_blocks": len(self.host_ref)}


def shared_prefix_groups(tables: Sequence[Sequence[int]], lens: Sequence[int], block_size: int,
                         max_members: int) -> List[Tuple[int, int, int]]:
    """Groups of consecutive batch rows that read the same full leading blocks.

    [P1] section 15 item 1: a full block referenced by several sequences is
    immutable, and its payload may be read by all of them at once.  A decode
    can then read such a block once for every sequence whose table holds it
    and combine that part of the attention with each sequence's own blocks
    ([P2] section 11: summaries of disjoint token sets merge exactly).  This
    function is the host rule that picks the groups; it fixes no arithmetic.

    Row n holds floor(lens[n] / B) full blocks.  Rows are walked in batch
    order.  A run starts at a row with L = its full-block count.  The next row
    joins the run when the run has fewer than ``max_members`` rows and the
    row's table starts with c >= 1 of the run's first L entries (c counted
    among the row's own full blocks) and joining does not lower the bytes the
    run saves: with k rows so far, k * c >= (k - 1) * L.  Then L becomes c.
    Otherwise the run closes and the row starts a new one.  Each closed run of
    at least 2 rows with L >= 1 is returned as (first row, rows, L * B shared
    tokens).
    """
    groups: List[Tuple[int, int, int]] = []
    n = len(lens)
    full = [max(int(s), 0) // block_size for s in lens]

    def close(first: int, count: int, shared_blocks: int) -> None:
        if count >= 2 and shared_blocks >= 1:
            groups.append((first, count, shared_blocks * block_size))

    if n == 0:
        return groups
    first, count, L = 0, 1, full[0]
    for row in range(1, n):
        c = 0
        limit = min(L, full[row])
        while c < limit and tables[row][c] == tables[first][c]:
            c += 1
        if count < max_members and c >= 1 and count * c >= (count - 1) * L:
            count += 1
            L = c
        else:
            close(first, count, L)
            first, count, L = row, 1, full[row]
    close(first, count, L)
    return groups


class PrefixCachingModel(BlockManagerModel):
    """The block manager with automatic prefix caching.

    What the pages fix ([P1] section 18; [P2] section 6; [P3] "Prefix
    caching"): a full block is identified by its tokens together with its
    whole preceding context, so equal text after a different prefix does not
    match; a block whose reference count drops to 0 stays cached and
    reusable, in an LRU structure; a request whose prefix matches takes the
    cached blocks (0 -> 1 when idle) instead of recomputing them; allocation
    under pressure reclaims idle cached blocks before it fails ([P1] section
    19).

    Readings where the pages leave details open:
      * A cached block is keyed by the exact token ids from the start of the
        sequence to its own end (its chain).  Only full blocks are cached; a
        lookup takes the longest run of leading full blocks whose chains are
        cached and stops at the first miss.  A block whose parent was evicted
        stays reachable: a request that recomputes the parent finds it again.
      * A block that fills up (a prompt's full blocks past the cached run, or
        a block filled through appends of known tokens) is cached then; if
        its chain is already cached in another block (a request that missed
        an evicted parent can meet its surviving child), it stays uncached.
        An append without a token id ends the sequence's chain: its later
        blocks are not cached.
      * Release walks the table from its last block to its first; a cached
        block reaching 0 joins the idle list at its most recent end, any
        other block the LIFO free list.  So a finished sequence's deepest
        blocks are evicted before its shallower ones.
      * Allocation takes the free list first, then evicts the least recently
        released idle block (its entry is dropped).
      * Batch appends check capacity first (a dry run of the copy-on-write
        decisions) and then cannot fail; nothing is undone.
    """

    def __init__(self, num_blocks: int, block_size: int, pop_order: Optional[Sequence[int]] = None):
        super().__init__(num_blocks, block_size, pop_order)
        self.index: Dict[Tuple[int, ...], int] = {}  # chain -> block
        self.entry: Dict[int, Tuple[int, ...]] = {}  # block -> chain
        self.idle: List[int] = []  # cached blocks with no reference, least recently released first
        self.tokens: Dict[int, Optional[List[int]]] = {}  # seq -> its token ids (None: some unknown)
        self.hit_blocks = 0
        self.evictions = 0

    # -- allocation with eviction -------------------------------------------
    def _available(self) -> int:
        return len(self.free) + len(self.idle)

    def _pop(self) -> int:
        if self.free:
            b = self.free.pop()
        else:
            b = self.idle.pop(0)  # least recently released
            del self.index[self.entry.pop(b)]
            self.evictions += 1
        self.ref[b] = 1
        return b

    def _take(self, b: int) -> None:
        """One more reference to a cached block (0 -> 1 leaves the idle list)."""
        if self.ref[b] == 0:
            self.idle.remove(b)
        self.ref[b] += 1

    # -- requests -------------------------------------------------------------
    def lookup(self, tokens: Sequence[int]) -> List[int]:
        """Blocks of the longest cached run of leading full blocks of `tokens` (no state change)."""
        B = self.block_size
        blocks = []
        for i in range(len(tokens) // B):
            b = self.index.get(tuple(int(t) for t in tokens[:(i + 1) * B]))
            if b is None:
                break
            blocks.append(b)
        return blocks

    def add_seq_tokens(self, seq: int, tokens: Sequence[int]) -> Tuple[int, int]:
        """A new sequence with these prompt token ids.  Returns (status, cached tokens reused)."""
        B = self.block_size
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        if n <= 0:
            return ERR_INVALID_ARG, 0
        if seq in self.tables:
            return ERR_EXISTS, 0
        hits = self.lookup(tokens)
        nblocks = -(-n // B)
        idle_hits = sum(1 for b in hits if self.ref[b] == 0)
        if self._available() - idle_hits < nblocks - len(hits):
            return ERR_NO_FREE_BLOCKS, 0
        table: List[int] = []
        for b in hits:
            self._take(b)
            table.append(b)
        self.hit_blocks += len(hits)
        for i in range(len(hits), nblocks):
            b = self._pop()
            table.append(b)
            key = tuple(tokens[:(i + 1) * B])
            if (i + 1) * B <= n and key not in self.index:  # a full block of the prompt: cache it
                self.index[key] = b
                self.entry[b] = key
        self.tables[seq] = table
        self.lens[seq] = n
        self.tokens[seq] = tokens
        return OK, len(hits) * B

    def add_seq(self, seq: int, num_tokens: int) -> int:
        st = super().add_seq(seq, num_tokens)
        if st == OK:  # no token ids: nothing of it can be cached
            self.tokens[seq] = None
        return st

    def fork(self, parent: int, child: int) -> int:
        st = super().fork(parent, child)
        if st == OK:
            t = self.tokens[parent]
            self.tokens[child] = None if t is None else list(t)
        return st

    def append_token(self, seq: int, token: Optional[int]) -> Tuple[int, int, int, int]:
        """append_slot, knowing the new token's id (None: unknown, which ends the chain)."""
        if seq not in self.tables:
            return ERR_NOT_FOUND, -1, -1, -1
        st, slot, src, dst = BlockManagerModel.append_slot(self, seq)
        if st != OK:
            return st, slot, src, dst
        t = self.tokens[seq]
        if token is None or t is None:
            self.tokens[seq] = None
        else:
            t.append(int(token))
            if len(t) % self.block_size == 0:  # the tail block is now full: cache it unless its chain is
                key = tuple(t)
                if key not in self.index:
                    b = self.tables[seq][-1]
                    self.index[key] = b
                    self.entry[b] = key
        return OK, slot, src, dst

    def append_slot(self, seq: int) -> Tuple[int, int, int, int]:
        return self.append_token(seq, None)

    def append_tokens(self, seqs: Sequence[int], tokens: Optional[Sequence[int]]):
        """Batch append, all-or-nothing by a capacity check first.  Returns (status, slots, cow_pairs, failed_index)."""
        for i, seq in enumerate(seqs):
            if seq not in self.tables:
                return ERR_NOT_FOUND, [], [], i
            if seq in self.swapped:
                return ERR_INVALID_ARG, [], [], i
        need, refs = 0, {}
        for i, seq in enumerate(seqs):
            if self.lens[seq] % self.block_size == 0:
                need += 1
            else:
                tail = self.tables[seq][-1]
                r = refs.get(tail, self.ref[tail])
                if r > 1:
                    need += 1
                    refs[tail] = r - 1
            if need > self._available():  # the append of seqs[i] would find no block
                return ERR_NO_FREE_BLOCKS, [], [], i
        slots, pairs = [], []
        for i, seq in enumerate(seqs):
            st, slot, src, dst = self.append_token(seq, None if tokens is None else tokens[i])
            assert st == OK
            slots.append(slot)
            if src >= 0:
                pairs.append((src, dst))
        return OK, slots, pairs, -1

    def append_slots(self, seqs: Sequence[int]):
        return self.append_tokens(seqs, None)

    def _release(self, b: int) -> None:
        (self.idle if b in self.entry else self.free).append(b)

    def free_seq(self, seq: int) -> int:
        if seq not in self.tables:
            return ERR_NOT_FOUND
        if seq in self.swapped:
            self._free_host(seq)
        else:
            for b in reversed(self.tables[seq]):
                self._unref(b)
            del self.tables[seq]
            del self.lens[seq]
        del self.tokens[seq]
        return OK

    def cached_prefix(self, b: int) -> List[int]:
        """The token ids a cached block stands for: the whole chain up to its end."""
        return list(self.entry[b])

    def stats(self) -> Dict[str, int]:
        s = super().stats()
        s["num_cached"] = len(self.entry)
        s["num_idle"] = len(self.idle)
        s["hit_blocks"] = self.hit_blocks
        s["evictions"] = self.evictions
        return s

// Host block manager: free list, per-block reference counts, block tables,
// fork, copy-on-write of a shared unaligned tail, release.
//
// Rules from "PagedAttention: Virtual Memory for the KV Cache": a sequence of
// S tokens holds ceil(S / B) blocks (section 8); fork duplicates the table and
// adds a reference per block (section 16); an append into a shared tail block
// clones it first (sections 15-16); release returns blocks whose count reaches
// zero to the free list (section 17); running out of blocks fails without
// changing anything (section 20, test 4).  The free list is a LIFO stack (the
// teaching allocator of section 20 pops from and pushes to the same end).
//
// Data structures are sized for large pools: a flat int32 refcount array, an
// int32 stack for the free list, and per-sequence vectors in a hash map.  All
// operations are O(1) amortised except fork/release (O(table length)) and
// stats (O(total table entries)).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
  // prefix cache: token ids of the partial tail block, the interned chain of
  // the full blocks before it (0: none), and whether all token ids of the
  // sequence are known
  std::vector<int32_t> pending;
  int64_t chain = 0;
  bool known = false;
  bool swapped = false;  // the table holds host block ids
};

// Hash of a full block's B token ids after the chain id of the tokens before
// it, for the chain index.  splitmix64's finaliser mixes each word in.  The
// hash only picks candidates: a match compares the parent chain id and the
// token ids exactly, so equal chain ids mean equal token chains.
uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

uint64_t chain_hash(uint64_t parent, const int32_t* tokens, int n) {
  uint64_t h = mix64(parent + 0x9e3779b97f4a7c15ull);
  for (int i = 0; i < n; ++i) h = mix64(h ^ static_cast<uint32_t>(tokens[i]) ^ (static_cast<uint64_t>(i + 1) << 32));
#ifdef PA_CHAIN_HASH_BITS  // test builds only: a hash this narrow makes distinct chains collide all the time
  h &= (uint64_t(1) << PA_CHAIN_HASH_BITS) - 1;
#endif
  return h;
}

struct Undo {  // what one append did, so a failed batch can be rolled back
  int64_t seq;
  int32_t cow_src;  // -1 when no copy-on-write happened
  int32_t cow_dst;
};

}  // namespace

struct pa_bm {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t cow_copies = 0;

  // ---- prefix cache (off unless enabled while no sequence exists) ----------
  // A token chain (the token ids of the leading full blocks of some sequence)
  // is interned: chain 0 is the empty chain, and chain c = (parent chain,
  // B token ids) is unique, so two requests share a prefix exactly when they
  // reach the same chain id.  A chain lives while something holds it: the
  // cached block that stands for it, a longer chain, or a sequence whose
  // tokens so far end with it.
  struct Chain {
    int64_t parent;
    int32_t block;  // the cached block holding these tokens, or -1
    int32_t refs;
  };
  bool caching = false;
  std::vector<uint8_t> cached;         // block holds a cached full block
  std::vector<int64_t> blk_chain;      // its chain
  std::vector<Chain> chains;           // [0] the empty chain
  std::vector<int32_t> chain_tokens;   // [chain][B]
  std::vector<int64_t> chain_free;     // ids to reuse
  std::unordered_multimap<uint64_t, int64_t> index;  // hash of (parent, tokens) -> chain
  int64_t num_cached = 0;
  // idle list: cached blocks without references, least recently released at the head
  std::vector<int32_t> idle_prev, idle_next;
  int32_t idle_head = -1, idle_tail = -1;
  int64_t idle_count = 0, hit_blocks = 0, evictions = 0;

  // ---- host pool for swapped-out sequences ---------------------------------
  std::vector<int32_t> host_free;  // top = back()
  std::vector<int32_t> host_ref;
  int64_t num_swapped = 0;

  int64_t available() const { return static_cast<int64_t>(free_stack.size()) + (caching ? idle_count : 0); }

  void idle_push(int32_t b) {  // most recently released end
    idle_prev[b] = idle_tail;
    idle_next[b] = -1;
    if (idle_tail >= 0) idle_next[idle_tail] = b; else idle_head = b;
    idle_tail = b;
    ++idle_count;
  }
  void idle_remove(int32_t b) {
    const int32_t p = idle_prev[b], n = idle_next[b];
    if (p >= 0) idle_next[p] = n; else idle_head = n;
    if (n >= 0) idle_prev[n] = p; else idle_tail = p;
    --idle_count;
  }

  // the chain (parent, tokens), or -1
  int64_t chain_find(int64_t parent, const int32_t* tokens) const {
    auto range = index.equal_range(chain_hash(static_cast<uint64_t>(parent), tokens, block_size));
    for (auto it = range.first; it != range.second; ++it) {
      const int64_t c = it->second;
      if (chains[c].parent == parent &&
          std::memcmp(&chain_tokens[static_cast<size_t>(c) * block_size], tokens, sizeof(int32_t) * block_size) == 0)
        return c;
    }
    return -1;
  }
  void chain_ref(int64_t c) {
    if (c > 0) ++chains[c].refs;
  }
  // one holder of chain c lets go; a chain no one holds is dropped, and lets go of its parent
  void chain_unref(int64_t c) {
    while (c > 0 && --chains[c].refs == 0) {
      auto range = index.equal_range(chain_hash(static_cast<uint64_t>(chains[c].parent),
                                                &chain_tokens[static_cast<size_t>(c) * block_size], block_size));
      for (auto it = range.first; it != range.second; ++it)
        if (it->second == c) {
          index.erase(it);
          break;
        }
      chain_free.push_back(c);
      c = chains[c].parent;
    }
  }
  // the chain (parent, tokens), made if it does not exist (it then holds its parent)
  int64_t chain_intern(int64_t parent, const int32_t* tokens) {
    const int64_t found = chain_find(parent, tokens);
    if (found >= 0) return found;
    int64_t c;
    if (!chain_free.empty()) {
      c = chain_free.back();
      chain_free.pop_back();
    } else {
      c = static_cast<int64_t>(chains.size());
      chains.push_back({});
      chain_tokens.resize(chain_tokens.size() + block_size);
    }
    chains[c] = {parent, -1, 0};
    std::memcpy(&chain_tokens[static_cast<size_t>(c) * block_size], tokens, sizeof(int32_t) * block_size);
    index.emplace(chain_hash(static_cast<uint64_t>(parent), tokens, block_size), c);
    chain_ref(parent);
    return c;
  }

  // the cached block holding (parent, tokens), or -1
  int32_t find(int64_t parent, const int32_t* tokens) const {
    const int64_t c = chain_find(parent, tokens);
    return c >= 0 ? chains[c].block : -1;
  }
  // cache block b as (parent, tokens) unless that chain is cached already; returns the chain
  int64_t remember(int32_t b, int64_t parent, const int32_t* tokens) {
    const int64_t c = chain_intern(parent, tokens);
    if (chains[c].block < 0) {
      chains[c].block = b;
      chain_ref(c);
      cached[b] = 1;
      blk_chain[b] = c;
      ++num_cached;
    }
    return c;
  }
  void forget(int32_t b) {
    const int64_t c = blk_chain[b];
    chains[c].block = -1;
    cached[b] = 0;
    --num_cached;
    chain_unref(c);
  }
  // sequence s's chain moves to c
  void set_chain(Seq& s, int64_t c) {
    chain_ref(c);
    chain_unref(s.chain);
    s.chain = c;
  }

  int32_t pop() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {  // evict the least recently released idle cached block
      b = idle_head;
      idle_remove(b);
      forget(b);
      ++evictions;
    }
    ref[b] = 1;
    return b;
  }

  void release(int32_t b) {  // a reference dropped to 0
    if (caching && cached[b]) idle_push(b); else free_stack.push_back(b);
  }

  // after an append of `token` (nullptr: unknown) to sequence s
  void note_token(Seq& s, const int32_t* token) {
    if (!caching) return;
    if (!token || !s.known) {
      s.known = false;
      s.pending.clear();
      set_chain(s, 0);
      return;
    }
    s.pending.push_back(*token);
    if (s.len % block_size == 0) {  // the tail block is full: cache it
      set_chain(s, remember(s.table.back(), s.chain, s.pending.data()));
      s.pending.clear();
    }
  }

  // Where position S of sequence s goes ("PagedAttention: Virtual Memory for
  // the KV Cache", sections 15-16): a fresh block when S is a multiple of B
  // (kOpen); a private copy of a partly filled tail that other sequences share,
  // since shared blocks are immutable (kClone); else the tail itself (kWrite).
  enum Placement { kOpen, kClone, kWrite };
  Placement placement(const Seq& s) const {
    if (s.len % block_size == 0) return kOpen;
    return ref[s.table.back()] > 1 ? kClone : kWrite;
  }

  // Reserve the slot of position S = len: checks first (nothing changes on an
  // error), then the whole effect.  Afterwards the sequence holds its last
  // block alone; a clone moves its reference from the shared tail to the copy.
  int append(int64_t id, int32_t* slot, int32_t* src, int32_t* dst) {
    *slot = -1;
    *src = -1;
    *dst = -1;
    auto it = seqs.find(id);
    if (it == seqs.end()) return PA_ERR_NOT_FOUND;
    Seq& s = it->second;
    if (s.swapped) return PA_ERR_INVALID_ARG;
    const Placement where = placement(s);
    if (where != kWrite && available() == 0) return PA_ERR_NO_FREE_BLOCKS;
    const int64_t S = s.len;
    if (where == kOpen) {
      s.table.push_back(pop());
    } else if (where == kClone) {
      const int32_t shared = s.table.back();
      const int32_t copy = pop();
      s.table.back() = copy;
      ref[shared] -= 1;  // still held by the other owners
      *src = shared;
      *dst = copy;
      ++cow_copies;
    }
    s.len = S + 1;
    *slot = s.table[S / block_size] * block_size + static_cast<int32_t>(S % block_size);
    return PA_OK;
  }

  void undo(const Undo& u) {
    Seq& s = seqs[u.seq];
    s.len -= 1;
    if (u.cow_src >= 0) {
      ref[u.cow_dst] = 0;
      free_stack.push_back(u.cow_dst);
      ref[u.cow_src] += 1;
      s.table.back() = u.cow_src;
      --cow_copies;
    } else if (s.len % block_size == 0) {
      const int32_t b = s.table.back();
      s.table.pop_back();
      ref[b] = 0;
      free_stack.push_back(b);
    }
  }
};

extern "C" {

pa_bm* pa_bm_create(int num_blocks, int block_size, const int32_t* pop_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return nullptr;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->free_stack.resize(num_blocks);
  if (pop_order) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = pop_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return nullptr;
      }
      seen[b] = 1;
      bm->free_stack[num_blocks - 1 - i] = b;  // first entry ends on top
    }
  } else {
    for (int i = 0; i < num_blocks; ++i) bm->free_stack[i] = num_blocks - 1 - i;
  }
  return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_add_seq(pa_bm* bm, int64_t seq, int num_tokens) {
  if (!bm || num_tokens <= 0) return PA_ERR_INVALID_ARG;
  if (bm->seqs.count(seq)) return PA_ERR_EXISTS;
  const int64_t need = (static_cast<int64_t>(num_tokens) + bm->block_size - 1) / bm->block_size;
  if (bm->available() < need) return PA_ERR_NO_FREE_BLOCKS;
  Seq s;
  s.table.reserve(need + 1);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->pop());
  s.len = num_tokens;
  s.known = false;  // no token ids: nothing of it is cached
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

int pa_bm_enable_prefix_cache(pa_bm* bm) {
  if (!bm || !bm->seqs.empty()) return PA_ERR_INVALID_ARG;
  if (bm->caching) return PA_OK;
  const size_t nb = static_cast<size_t>(bm->num_blocks);
  bm->cached.assign(nb, 0);
  bm->blk_chain.assign(nb, 0);
  bm->chains.assign(1, {0, -1, 0});  // the empty chain
  bm->chain_tokens.assign(static_cast<size_t>(bm->block_size), 0);
  bm->idle_prev.assign(nb, -1);
  bm->idle_next.assign(nb, -1);
  bm->caching = true;
  return PA_OK;
}

int pa_bm_add_seq_tokens(pa_bm* bm, int64_t seq, const int32_t* tokens, int num_tokens, int* cached_tokens) {
  if (!bm || num_tokens <= 0 || !tokens) return PA_ERR_INVALID_ARG;
  if (cached_tokens) *cached_tokens = 0;
  if (bm->seqs.count(seq)) return PA_ERR_EXISTS;
  if (!bm->caching) return pa_bm_add_seq(bm, seq, num_tokens);
  const int B = bm->block_size;
  const int64_t nblocks = (static_cast<int64_t>(num_tokens) + B - 1) / B;
  const int64_t full = num_tokens / B;
  // the longest run of leading full blocks whose chains are cached (no change yet)
  std::vector<int32_t> hits;
  int64_t parent = 0;
  int64_t idle_hits = 0;
  for (int64_t i = 0; i < full; ++i) {
    const int32_t b = bm->find(parent, tokens + i * B);
    if (b < 0) break;
    hits.push_back(b);
    if (bm->ref[b] == 0) ++idle_hits;
    parent = bm->blk_chain[b];
  }
  if (bm->available() - idle_hits < nblocks - static_cast<int64_t>(hits.size())) return PA_ERR_NO_FREE_BLOCKS;
  Seq s;
  s.table.reserve(nblocks + 1);
  for (int32_t b : hits) {  // reuse: 0 -> 1 leaves the idle list
    if (bm->ref[b] == 0) bm->idle_remove(b);
    bm->ref[b] += 1;
    s.table.push_back(b);
  }
  bm->hit_blocks += static_cast<int64_t>(hits.size());
  for (int64_t i = static_cast<int64_t>(hits.size()); i < nblocks; ++i) {
    const int32_t b = bm->pop();
    s.table.push_back(b);
    if (i < full) parent = bm->remember(b, parent, tokens + i * B);  // a full block of the prompt
  }
  s.len = num_tokens;
  s.chain = 0;
  bm->set_chain(s, parent);
  s.known = true;
  s.pending.assign(tokens + full * B, tokens + num_tokens);
  bm->seqs.emplace(seq, std::move(s));
  if (cached_tokens) *cached_tokens = static_cast<int>(hits.size()) * B;
  return PA_OK;
}

int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  if (bm->seqs.count(child)) return PA_ERR_EXISTS;
  if (it->second.swapped) return PA_ERR_INVALID_ARG;
  Seq s = it->second;  // copy of the table; no data moves
  for (int32_t b : s.table) bm->ref[b] += 1;
  if (bm->caching) bm->chain_ref(s.chain);  // the child's tokens end with the same chain
  bm->seqs.emplace(child, std::move(s));
  return PA_OK;
}

int pa_bm_append_slot(pa_bm* bm, int64_t seq, int32_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PA_ERR_INVALID_ARG;
  const int st = bm->append(seq, slot, cow_src, cow_dst);
  if (st == PA_OK) bm->note_token(bm->seqs[seq], nullptr);
  return st;
}

// Batch append with a prefix cache: existence, then a dry run of the blocks
// the appends take (fresh blocks and copy-on-write, with the reference
// counts the earlier appends of the batch leave), then the appends, which
// cannot fail.  tokens (nullable) are the appended token ids.
static int append_batch_cached(pa_bm* bm, const int64_t* seqs, const int32_t* tokens, int n, int32_t* slots,
                               int32_t* cow_pairs, int* num_pairs) {
  std::vector<Seq*> rows(n);
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || it->second.swapped) {
      *num_pairs = -i - 1;
      return it == bm->seqs.end() ? PA_ERR_NOT_FOUND : PA_ERR_INVALID_ARG;
    }
    rows[i] = &it->second;
  }
  std::unordered_map<int32_t, int32_t> refs;  // tail block -> references left by earlier appends
  int64_t need = 0;
  for (int i = 0; i < n; ++i) {
    const Seq& s = *rows[i];
    if (s.len % bm->block_size == 0) {
      ++need;
    } else {
      const int32_t tail = s.table.back();
      auto r = refs.find(tail);
      const int32_t cur = r == refs.end() ? bm->ref[tail] : r->second;
      if (cur > 1) {
        ++need;
        refs[tail] = cur - 1;
      }
    }
    if (need > bm->available()) {
      *num_pairs = -i - 1;
      return PA_ERR_NO_FREE_BLOCKS;
    }
  }
  int pairs = 0;
  for (int i = 0; i < n; ++i) {
    int32_t slot, src, dst;
    bm->append(seqs[i], &slot, &src, &dst);  // checked above: cannot fail
    bm->note_token(*rows[i], tokens ? tokens + i : nullptr);
    slots[i] = slot;
    if (src >= 0) {
      cow_pairs[2 * pairs] = src;
      cow_pairs[2 * pairs + 1] = dst;
      ++pairs;
    }
  }
  *num_pairs = pairs;
  return PA_OK;
}

int pa_bm_append_tokens(pa_bm* bm, const int64_t* seqs, const int32_t* tokens, int n, int32_t* slots,
                        int32_t* cow_pairs, int* num_pairs) {
  if (!bm || n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_pairs) return PA_ERR_INVALID_ARG;
  if (!bm->caching) return pa_bm_append_slots(bm, seqs, n, slots, cow_pairs, num_pairs);
  return append_batch_cached(bm, seqs, tokens, n, slots, cow_pairs, num_pairs);
}

int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, int n, int32_t* slots, int32_t* cow_pairs,
                       int* num_pairs) {
  if (!bm || n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_pairs)
    return PA_ERR_INVALID_ARG;
  if (bm->caching) return append_batch_cached(bm, seqs, nullptr, n, slots, cow_pairs, num_pairs);
  std::vector<Undo> done;
  done.reserve(n);
  int pairs = 0;
  for (int i = 0; i < n; ++i) {
    int32_t slot, src, dst;
    const int st = bm->append(seqs[i], &slot, &src, &dst);
    if (st != PA_OK) {
      for (auto u = done.rbegin(); u != done.rend(); ++u) bm->undo(*u);
      *num_pairs = -i - 1;
      return st;
    }
    done.push_back({seqs[i], src, dst});
    slots[i] = slot;
    if (src >= 0) {
      cow_pairs[2 * pairs] = src;
      cow_pairs[2 * pairs + 1] = dst;
      ++pairs;
    }
  }
  *num_pairs = pairs;
  return PA_OK;
}

int pa_bm_free_seq(pa_bm* bm, int64_t seq) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  const std::vector<int32_t>& t = it->second.table;
  if (it->second.swapped) {  // host blocks
    for (int32_t hb : t)
      if (--bm->host_ref[hb] == 0) bm->host_free.push_back(hb);
    --bm->num_swapped;
  } else if (bm->caching) {  // last block first: a sequence's deepest blocks become the oldest idle entries
    for (auto b = t.rbegin(); b != t.rend(); ++b)
      if (--bm->ref[*b] == 0) bm->release(*b);
  } else {
    for (int32_t b : t)
      if (--bm->ref[b] == 0) bm->free_stack.push_back(b);
  }
  if (bm->caching) bm->chain_unref(it->second.chain);
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_build_batch(pa_bm* bm, const int64_t* seqs, int n, int max_blocks_per_seq,
                      int32_t* block_tables_out, int32_t* context_lens_out) {
  if (!bm || n < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  if (n > 0 && (!seqs || !context_lens_out || (max_blocks_per_seq > 0 && !block_tables_out)))
    return PA_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {  // validate everything before writing anything
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
    if (it->second.swapped) return PA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks_per_seq) return PA_ERR_INVALID_ARG;
    if (it->second.len > INT32_MAX) return PA_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = block_tables_out + static_cast<int64_t>(i) * max_blocks_per_seq;
    const size_t nb = s.table.size();
    if (nb) std::memcpy(row, s.table.data(), nb * sizeof(int32_t));
    for (int64_t j = nb; j < max_blocks_per_seq; ++j) row[j] = 0;
    context_lens_out[i] = static_cast<int32_t>(s.len);
  }
  return PA_OK;
}

int pa_bm_shared_groups(pa_bm* bm, const int64_t* seqs, int n, int max_members, int32_t* groups_out, int cap,
                        int* num_groups) {
  if (!bm || n < 0 || max_members < 1 || cap < 0 || !num_groups) return PA_ERR_INVALID_ARG;
  if (n > 0 && !seqs) return PA_ERR_INVALID_ARG;
  std::vector<const Seq*> rows(n);
  for (int i = 0; i < n; ++i) {  // validate everything before writing anything
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
    if (it->second.swapped) return PA_ERR_INVALID_ARG;
    rows[i] = &it->second;
  }
  const int64_t B = bm->block_size;
  auto full = [&](int i) { return rows[i]->len / B; };  // full blocks of row i
  // Greedy runs in batch order: a row joins the run while the run has room,
  // the row starts with c >= 1 of the run's L shared full blocks, and joining
  // keeps the bytes saved (k * c >= (k - 1) * L for k rows so far).
  std::vector<int32_t> found;
  auto close = [&](int first, int count, int64_t shared_blocks) {
    if (count >= 2 && shared_blocks >= 1) {
      found.push_back(first);
      found.push_back(count);
      found.push_back(static_cast<int32_t>(shared_blocks * B));
    }
  };
  if (n > 0) {
    int first = 0, count = 1;
    int64_t L = full(0);
    for (int i = 1; i < n; ++i) {
      const int64_t limit = std::min(L, full(i));
      const std::vector<int32_t>& a = rows[first]->table;
      const std::vector<int32_t>& b = rows[i]->table;
      int64_t c = 0;
      while (c < limit && a[c] == b[c]) ++c;
      if (count < max_members && c >= 1 && static_cast<int64_t>(count) * c >= static_cast<int64_t>(count - 1) * L) {
        ++count;
        L = c;
      } else {
        close(first, count, L);
        first = i;
        count = 1;
        L = full(i);
      }
    }
    close(first, count, L);
  }
  const int g = static_cast<int>(found.size() / 3);
  *num_groups = g;
  if (g > cap || (g > 0 && !groups_out)) return PA_ERR_INVALID_ARG;
  if (g > 0) std::memcpy(groups_out, found.data(), found.size() * sizeof(int32_t));
  return PA_OK;
}

int pa_bm_refcount(pa_bm* bm, int block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int pa_bm_num_free(pa_bm* bm) { return bm ? static_cast<int>(bm->free_stack.size()) : -1; }

int64_t pa_bm_seq_len(pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int pa_bm_block_table(pa_bm* bm, int64_t seq, int32_t* out, int cap, int* n_out) {
  if (!bm || !n_out || cap < 0) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  const auto& t = it->second.table;
  *n_out = static_cast<int>(t.size());
  if (static_cast<int64_t>(t.size()) > cap || (!out && !t.empty())) return PA_ERR_INVALID_ARG;
  if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  return PA_OK;
}

int pa_bm_free_list(pa_bm* bm, int32_t* out, int cap, int* n_out) {
  if (!bm || !n_out || cap < 0) return PA_ERR_INVALID_ARG;
  const int64_t n = static_cast<int64_t>(bm->free_stack.size());
  *n_out = static_cast<int>(n);
  if (n > cap || (!out && n > 0)) return PA_ERR_INVALID_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = bm->free_stack[n - 1 - i];
  return PA_OK;
}

int pa_bm_can_allocate(pa_bm* bm, int num_tokens) {
  if (!bm || num_tokens <= 0) return 0;
  const int64_t need = (static_cast<int64_t>(num_tokens) + bm->block_size - 1) / bm->block_size;
  return bm->available() >= need ? 1 : 0;
}

int pa_bm_stats(pa_bm* bm, pa_bm_stats_t* out) {
  if (!bm || !out) return PA_ERR_INVALID_ARG;
  // fill of a block = valid tokens it holds; sharers of a block agree on it,
  // take the largest over the sequences that reference it
  std::vector<int32_t> fill(bm->num_blocks, 0);
  for (const auto& kv : bm->seqs) {
    const Seq& s = kv.second;
    if (s.swapped) continue;  // host blocks are not part of the device pool
    for (size_t lb = 0; lb < s.table.size(); ++lb) {
      const int64_t valid = s.len - static_cast<int64_t>(lb) * bm->block_size;
      const int32_t v = static_cast<int32_t>(valid < bm->block_size ? valid : bm->block_size);
      int32_t& f = fill[s.table[lb]];
      if (v > f) f = v;
    }
  }
  int64_t used = 0, stored = 0;
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->ref[b] > 0) ++used;
    stored += fill[b];
  }
  out->num_blocks = bm->num_blocks;
  out->num_free = static_cast<int64_t>(bm->free_stack.size());
  out->num_used = used;
  out->num_seqs = static_cast<int64_t>(bm->seqs.size());
  out->cow_copies = bm->cow_copies;
  out->stored_tokens = stored;
  out->tail_waste_slots = used * bm->block_size - stored;
  return PA_OK;
}

int pa_bm_enable_host_pool(pa_bm* bm, int num_host_blocks, const int32_t* pop_order) {
  if (!bm || num_host_blocks <= 0 || !bm->host_ref.empty()) return PA_ERR_INVALID_ARG;
  std::vector<int32_t> stack(num_host_blocks);
  if (pop_order) {
    std::vector<uint8_t> seen(num_host_blocks, 0);
    for (int i = 0; i < num_host_blocks; ++i) {
      const int32_t b = pop_order[i];
      if (b < 0 || b >= num_host_blocks || seen[b]) return PA_ERR_INVALID_ARG;
      seen[b] = 1;
      stack[num_host_blocks - 1 - i] = b;  // first entry ends on top
    }
  } else {
    for (int i = 0; i < num_host_blocks; ++i) stack[i] = num_host_blocks - 1 - i;
  }
  bm->host_free = std::move(stack);
  bm->host_ref.assign(num_host_blocks, 0);
  return PA_OK;
}

// The listed sequences' distinct blocks in order of first appearance
// (sequence order, then table order), with the references they hold.
static int swap_prepare(pa_bm* bm, const int64_t* seqs, int n, bool want_swapped, std::vector<Seq*>& rows,
                        std::vector<int32_t>& blocks, std::vector<int32_t>& counts) {
  if (bm->host_ref.empty()) return PA_ERR_INVALID_ARG;
  std::unordered_map<int64_t, int> ids;
  rows.resize(n);
  for (int i = 0; i < n; ++i) {
    if (!ids.emplace(seqs[i], i).second) return PA_ERR_INVALID_ARG;  // listed twice
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
    if (it->second.swapped != want_swapped) return PA_ERR_INVALID_ARG;
    rows[i] = &it->second;
  }
  std::unordered_map<int32_t, int32_t> pos;
  for (Seq* s : rows)
    for (int32_t b : s->table) {
      auto r = pos.emplace(b, static_cast<int32_t>(blocks.size()));
      if (r.second) {
        blocks.push_back(b);
        counts.push_back(0);
      }
      ++counts[r.first->second];
    }
  return PA_OK;
}

int pa_bm_swap_out(pa_bm* bm, const int64_t* seqs, int n, int32_t* pairs_out, int cap, int* num_pairs) {
  if (!bm || n < 0 || (n > 0 && !seqs) || cap < 0 || !num_pairs) return PA_ERR_INVALID_ARG;
  std::vector<Seq*> rows;
  std::vector<int32_t> blocks, counts;
  int st = swap_prepare(bm, seqs, n, false, rows, blocks, counts);
  if (st != PA_OK) return st;
  const int need = static_cast<int>(blocks.size());
  *num_pairs = need;
  if (need > cap || (need > 0 && !pairs_out)) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(bm->host_free.size()) < need) return PA_ERR_NO_FREE_BLOCKS;
  std::unordered_map<int32_t, int32_t> where;
  for (int k = 0; k < need; ++k) {
    const int32_t b = blocks[k];
    const int32_t hb = bm->host_free.back();
    bm->host_free.pop_back();
    bm->host_ref[hb] = counts[k];
    bm->ref[b] -= counts[k];
    if (bm->ref[b] == 0) bm->release(b);  // other holders keep the device block
    pairs_out[2 * k] = b;
    pairs_out[2 * k + 1] = hb;
    where[b] = hb;
  }
  for (Seq* s : rows) {
    for (int32_t& b : s->table) b = where[b];
    s->swapped = true;
  }
  bm->num_swapped += n;
  return PA_OK;
}

int pa_bm_swap_in(pa_bm* bm, const int64_t* seqs, int n, int32_t* pairs_out, int cap, int* num_pairs) {
  if (!bm || n < 0 || (n > 0 && !seqs) || cap < 0 || !num_pairs) return PA_ERR_INVALID_ARG;
  std::vector<Seq*> rows;
  std::vector<int32_t> blocks, counts;
  int st = swap_prepare(bm, seqs, n, true, rows, blocks, counts);
  if (st != PA_OK) return st;
  const int need = static_cast<int>(blocks.size());
  *num_pairs = need;
  if (need > cap || (need > 0 && !pairs_out)) return PA_ERR_INVALID_ARG;
  if (bm->available() < need) return PA_ERR_NO_FREE_BLOCKS;
  std::unordered_map<int32_t, int32_t> where;
  for (int k = 0; k < need; ++k) {
    const int32_t hb = blocks[k];
    const int32_t b = bm->pop();
    bm->ref[b] = counts[k];
    bm->host_ref[hb] -= counts[k];
    if (bm->host_ref[hb] == 0) bm->host_free.push_back(hb);
    pairs_out[2 * k] = hb;
    pairs_out[2 * k + 1] = b;
    where[hb] = b;
  }
  for (Seq* s : rows) {
    for (int32_t& hb : s->table) hb = where[hb];
    s->swapped = false;
  }
  bm->num_swapped -= n;
  return PA_OK;
}

int pa_bm_swap_stats(pa_bm* bm, int64_t* num_swapped, int64_t* host_free, int64_t* host_blocks) {
  if (!bm || !num_swapped || !host_free || !host_blocks) return PA_ERR_INVALID_ARG;
  *num_swapped = bm->num_swapped;
  *host_free = static_cast<int64_t>(bm->host_free.size());
  *host_blocks = static_cast<int64_t>(bm->host_ref.size());
  return PA_OK;
}

int pa_bm_cache_stats(pa_bm* bm, pa_bm_cache_stats_t* out) {
  if (!bm || !out) return PA_ERR_INVALID_ARG;
  out->enabled = bm->caching ? 1 : 0;
  out->num_cached = bm->num_cached;
  out->num_idle = bm->idle_count;
  out->hit_blocks = bm->hit_blocks;
  out->evictions = bm->evictions;
  return PA_OK;
}

int pa_bm_idle_list(pa_bm* bm, int32_t* out, int cap, int* n_out) {
  if (!bm || !n_out || cap < 0) return PA_ERR_INVALID_ARG;
  *n_out = static_cast<int>(bm->idle_count);
  if (bm->idle_count > cap || (!out && bm->idle_count > 0)) return PA_ERR_INVALID_ARG;
  int i = 0;
  for (int32_t b = bm->idle_head; b >= 0; b = bm->idle_next[b]) out[i++] = b;
  return PA_OK;
}

}  // extern "C"

"""Oracle for PagedAttention decode: plain, slow, obviously correct CPU code.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP kernels, the
C ABI library, the Python binding) imports, links or calls this package; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the GPU path: no kernels,
headers, helpers, tables or layout conversion.  It works on the *logical* KV
pool ``[num_blocks][num_kv_heads][block_size][d_head]`` and never sees the
GPU's physical layout.

Modules
-------
attention      fp64 paged decode attention (gather through the block table,
               then softmax(q.K^T * scale).V), a separate dense attention
               routine, the per-block (m, z, u) summaries and their merge,
               address translation, and the append / block-copy storage rules.
block_manager  pure-Python block manager: LIFO free list, per-block reference
               counts, block tables, fork, copy-on-write of a shared tail
               block, release, batch building, the rule that groups
               consecutive batch rows sharing full leading blocks, and a
               prefix-caching variant (full blocks cached by their exact
               token chain, idle LRU, revival, eviction under pressure), and
               swapping of sequences to a host block pool and back.
fp8            KV cache held as FP8 E4M3 codes with per-(block, KV head)
               scales: code values, the saturating round-to-nearest-even
               quantizer, the quantizing append, block copy with scales, and
               decode over the dequantized cache.
int8           KV cache held as signed 8-bit integer codes with per-(block,
               KV head) scales: code values, the clamped round-half-to-even
               quantizer, the quantizing append, block copy with scales, and
               decode over the dequantized cache.
sizing         KV sizing, block-table footprint, tail waste and capacity
               arithmetic.

Sources (the three pages this work is built from):
  [P1] "PagedAttention: Virtual Memory for the KV Cache", int8ai.pages.dev,
       Module 02 Ch. 5.
  [P2] "PagedAttention in vLLM: scattered memory, exact attention",
       abhiram1809.github.io.
  [P3] "PagedAttention and KV Memory", blog.michaelsam94.com.

Every function is pinned by ``tests/test_oracle_*.py`` to values the pages
print, closed forms, special cases or invariants; none is "parity unpinned".
"""

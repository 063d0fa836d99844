/*
 * pa.h -- PagedAttention decode on AMD Instinct MI355X (gfx950): C ABI of libpa.so
 *
 * The KV cache of every sequence lives in fixed-size physical blocks of a
 * shared pool and is reached through a per-sequence block table of int32
 * physical block ids ("PagedAttention: Virtual Memory for the KV Cache",
 * sections 5-7).  One query token per sequence attends over its cache
 * (same page, section 1; "PagedAttention in vLLM: scattered memory, exact
 * attention", section 10).
 *
 * Conventions for every entry point
 *   - Array arguments of the device entry points (pa_decode, pa_append_kv,
 *     pa_copy_blocks) are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps device memory.  Block-manager (pa_bm_*)
 *     arguments are HOST pointers owned by the caller.
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t passed
 *     as void*; NULL = the default stream) and is ordered with other work on
 *     that stream only.  Within one decode step call pa_copy_blocks, then
 *     pa_append_kv, then pa_decode, on one stream.
 *   - Every entry point returns an int status (PA_OK = 0).  Argument errors
 *     are detected on the host before anything is enqueued and leave all
 *     state unchanged.  A fault inside a kernel surfaces at the caller's next
 *     synchronisation.  No C++ exception crosses the ABI.
 *   - All sizes are in elements unless a name ends in _bytes.
 *
 * Pool layout (one layer; a multi-layer pool stacks layers with a stride of
 * layer_stride_elems elements).  B = block_size, D = d_head; K and V pools
 * alike, every element type (fp32, bf16, or one-byte codes):
 *
 *   [num_blocks][Hkv][B][D]
 *       key element d of the token in slot `off` of block `pb`, KV head j:
 *       k_pool[((pb * Hkv + j) * B + off) * D + d]
 *       value element d: v_pool[((pb * Hkv + j) * B + off) * D + d]
 *
 *   Each (block, KV head) is one contiguous run of B * D * E bytes (E the
 *   element size) in each pool, its B token rows of D contiguous elements
 *   ("PagedAttention: Virtual Memory for the KV Cache", section 12 leaves the
 *   in-block layout to the implementation).  The decode kernels copy whole
 *   rows into LDS with 16-byte loads and form their matrix-core operands there
 *   (the value operand with gfx950's transposing LDS reads); the appends store
 *   each new row with 16-byte stores.
 *
 * Address translation ("PagedAttention: Virtual Memory for the KV Cache",
 * section 7): token i of a sequence lives in logical block i / B at offset
 * i % B, i.e. physical block block_table[i / B]; its slot is
 * block_table[i / B] * B + i % B.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes and element types ------------------------------------ */
enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,    /* bad pointer, size or combination of sizes           */
  PA_ERR_UNSUPPORTED = 2,    /* valid request outside the compiled shapes/dtypes    */
  PA_ERR_NO_FREE_BLOCKS = 3, /* pool exhausted; the operation changed nothing       */
  PA_ERR_EXISTS = 4,         /* sequence id already present                        */
  PA_ERR_NOT_FOUND = 5,      /* sequence id unknown                                 */
  PA_ERR_WORKSPACE = 6,      /* workspace missing or smaller than required          */
  PA_ERR_HIP = 7             /* the HIP runtime refused a launch                    */
};

/* PA_FP8_E4M3 and PA_INT8 name caches of one-byte codes (see pa_decode_fp8,
 * pa_decode_int8); queries, outputs and new tokens stay bf16 there. */
enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2, PA_INT8 = 3 };

/* Text for a status code (static storage; never NULL). */
const char* pa_status_string(int status);

/* Library ABI version; bumped on any incompatible change. */
int pa_version(void);

/* ---- decode attention ------------------------------------------------------
 *
 * pa_decode: one decode step of paged attention for a batch of sequences.
 * Defined by "PagedAttention: Virtual Memory for the KV Cache", sections 1
 * and 13, and "PagedAttention in vLLM: scattered memory, exact attention",
 * sections 10-11.  For sequence n, query head h, KV head j = h / (Hq / Hkv)
 * and tokens t < S = context_lens[n]:
 *
 *     s_t = scale * dot(q[n][h], K_t),  K_t, V_t gathered through the table
 *     out[n][h] = sum_t exp(s_t - max s) V_t / sum_t exp(s_t - max s)
 *
 * The work is split across the GPU in pieces of a sequence's context; each
 * piece that does not cover its whole sequence leaves a (max, shifted weight
 * sum, shifted value sum) summary in `workspace`, and a second kernel merges
 * the pieces of a sequence with the common-maximum rule of the second page,
 * section 11.  The split and the merge order are fixed for given sizes,
 * context_lens and device, so repeated calls on the same inputs give
 * bit-identical outputs.
 *
 *   out            [num_seqs][Hq][d_head], element type `dtype`
 *   q              [num_seqs][Hq][d_head], element type `dtype`
 *   k_pool, v_pool one layer's pools in the layout above, `num_blocks` blocks
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]; entries at logical
 *                  blocks >= ceil(S / B) are never read
 *   context_lens   int32 [num_seqs], 0 <= S <= max_context_len and
 *                  ceil(S / B) <= max_blocks_per_seq.  S = 0 gives zeros.
 *   scale          multiplies q.K (1 / sqrt(d_head) for the textbook rule)
 *   max_context_len an upper bound of all S (sizes the launch without a
 *                  device read)
 *   workspace      device scratch of at least pa_decode_workspace_bytes(...)
 *                  bytes; may be NULL when that size is 0.  Its contents
 *                  need no initialisation: a call writes every word of it
 *                  that the call reads.  Calls that may overlap in time need
 *                  separate workspaces.
 * Supported: Hq % Hkv == 0, Hq / Hkv <= 64, d_head in {64, 128},
 * block_size in {8, 16, 32}, dtype PA_F32 or PA_BF16 (fp32 accumulation;
 * bf16 outputs are rounded to nearest even).  Block ids outside
 * [0, num_blocks) are never dereferenced: the tokens they hold are left out
 * of the softmax.  num_blocks >= 1 and max_blocks_per_seq >= 1 when
 * num_seqs > 0.
 */
int pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* context_lens,
              int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
              int max_blocks_per_seq, int max_context_len, int num_blocks, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode_partitioned: pa_decode computed by the partitioned kernels -- the
 * shape of "PagedAttention: Virtual Memory for the KV Cache", section 13: one
 * workgroup per (partition of `partition_tokens` tokens, KV head, sequence)
 * looping over the partition's blocks, a summary per partition in
 * `workspace`, and a second kernel that merges the partitions of a sequence
 * in order ("PagedAttention in vLLM: scattered memory, exact attention",
 * section 11).  pa_decode itself takes this path for shapes the persistent
 * kernel does not serve (fp32, Hq / Hkv > 16, more than 3072 sequences);
 * this entry point takes it for every shape pa_decode supports.
 *   partition_tokens  0 = the size pa_decode would pick
 *                     (pa_decode_partition_tokens); else a multiple of 128
 *                     spanning at most 64 blocks (<= 64 * block_size);
 *                     anything else is PA_ERR_INVALID_ARG
 *   workspace         at least pa_decode_partitioned_workspace_bytes(...)
 *                     bytes (0, and NULL allowed, when every sequence fits
 *                     one partition); no initialisation needed
 * Every other argument, the outputs and the errors are those of pa_decode.
 */
int pa_decode_partitioned(void* out, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                          int max_blocks_per_seq, int max_context_len, int num_blocks, int dtype,
                          int partition_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pa_decode_partitioned needs for these sizes (0 for an
 * invalid combination or when no sequence spans two partitions). */
size_t pa_decode_partitioned_workspace_bytes(int num_seqs, int Hq, int Hkv, int d_head, int block_size,
                                             int max_context_len, int dtype, int partition_tokens);

/* pa_check_batch: validate a batch's lengths and block tables on the device,
 * against the sizes a decode call would be given.  The decode kernels trust
 * them for speed: a block id outside [0, num_blocks) is never dereferenced
 * but its tokens silently leave the softmax, and tokens past
 * max_blocks_per_seq * B are dropped.  This call makes such inputs visible
 * without a host copy of the tables ("PagedAttention: Virtual Memory for the
 * KV Cache", section 7: token i lives in physical block block_table[i / B];
 * section 8: the table holds int32 ids of pool blocks).  It enqueues one
 * kernel on `stream` that reads only context_lens[0 .. num_seqs) and the
 * table entries below each row's ceil(S / B), and writes
 *
 *   status[0]  rows with S < 0, S > max_context_len or
 *              ceil(S / B) > max_blocks_per_seq
 *   status[1]  table entries outside [0, num_blocks), among the first
 *              ceil(S / B) entries of every other row
 *   status[2]  the lowest row counted in status[0], -1 when none
 *   status[3]  the lowest row holding an entry counted in status[1], -1 when none
 *
 *   block_tables  int32 [num_seqs][max_blocks_per_seq], device
 *   context_lens  int32 [num_seqs], device
 *   status        int32 [4], device (or pinned host memory mapped for the
 *                 device); every word is written, nothing needs clearing
 * The batch is valid for pa_decode with these sizes iff status[0] and
 * status[1] are 0 once the stream reaches this point.  Errors (host, before
 * any launch): PA_ERR_INVALID_ARG for num_seqs < 0, max_blocks_per_seq < 1,
 * max_context_len < 0, num_blocks < 0, block_size < 1 or a NULL pointer the
 * call needs.  For pa_decode_step call it before the step (the step then
 * moves each row forward by one token). */
int pa_check_batch(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                   int max_blocks_per_seq, int max_context_len, int num_blocks, int block_size,
                   int32_t* status, void* stream);

/* pa_check_pairs: validate a list of copy-on-write pairs on the device before
 * pa_copy_blocks* ("PagedAttention: Virtual Memory for the KV Cache", sections
 * 15-16: a copy clones a shared block into a fresh block).  The copy kernels
 * assume what the block manager guarantees: no destination is named twice and
 * no destination is also a source in the same call (else the result depends on
 * the order the copies run in); a pair with an id outside [0, num_blocks) is
 * skipped.  One kernel on `stream` reads the pairs and writes
 *
 *   status[0]  pairs with an id outside [0, num_blocks)
 *   status[1]  pairs naming a destination that an earlier pair names
 *              (pairs naming it minus one, summed over destinations)
 *   status[2]  pairs whose destination is also some pair's source
 *   status[3]  the lowest index of a pair counted in status[0] or status[2], or
 *              naming a destination that another pair names; -1 when none
 *
 *   src_dst_pairs  int32 [num_pairs][2], device-readable
 *   status         int32 [4], device; every word is written
 * The pairs are valid for pa_copy_blocks* iff status[0..2] are 0.  Errors
 * (host, before any launch): PA_ERR_INVALID_ARG for num_pairs < 0,
 * num_blocks < 0 or a NULL pointer the call needs; PA_ERR_UNSUPPORTED for
 * num_blocks > 524288 (the check keeps two bitmaps of the pool in LDS). */
int pa_check_pairs(const int32_t* src_dst_pairs, int num_pairs, int num_blocks, int32_t* status, void* stream);

/* pa_decode_step: one whole decode step of the batch.  Each row attends to
 * its S cached tokens and to its new token (key and value from k_new / v_new,
 * at position S); then the new token is stored and the row moved forward
 * exactly as pa_append_step does ("PagedAttention: Virtual Memory for the KV
 * Cache", sections 13 and 16; "PagedAttention in vLLM: scattered memory,
 * exact attention", sections 10-11).  The attention takes the new token from
 * k_new / v_new, so its store does not have to finish first.  For row n with
 * S = context_lens[n] on entry and slot = slot_mapping[n]:
 *
 *     out[n] = attention of q[n] over the S cached tokens and the new token;
 *     when slot is the row's next position -- inside the pool, slot % B ==
 *     S % B and S / B < max_blocks_per_seq -- the new token's K/V are
 *     stored at slot, block_tables[n][S / B] = slot / B and
 *     context_lens[n] = S + 1; otherwise nothing is stored or changed.
 *
 * Where every row's slot is its next position this is, bit for bit,
 * pa_append_step followed by pa_decode.
 *
 *   k_new, v_new   [num_seqs][Hkv][d_head], element type `dtype`, device
 *   slot_mapping   int32 [num_seqs]; device-readable (device memory, or
 *                  pinned host memory mapped for the device)
 *   block_tables, context_lens   as for pa_decode, updated in place
 *   max_context_len an upper bound of S + 1
 * Other arguments, the workspace (pa_decode_workspace_bytes) and the errors
 * as for pa_decode.  Served for bf16, Hq / Hkv <= 16, num_seqs <= 3072 (the
 * persistent kernel); other shapes return PA_ERR_UNSUPPORTED and take
 * pa_append_step + pa_decode.
 */
int pa_decode_step(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                   const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens, int num_seqs,
                   int Hq, int Hkv, int d_head, int block_size, float scale, int max_blocks_per_seq,
                   int max_context_len, int num_blocks, int dtype, void* workspace, size_t workspace_bytes,
                   void* stream);

/* pa_decode_step_noalloc: pa_decode_step for callers that cannot allocate
 * device memory -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, outputs, row updates and
 * errors as pa_decode_step, without `workspace` / `workspace_bytes`: the
 * workspace is a fixed device array of PA_NOALLOC_SCRATCH_BYTES bytes inside
 * the library, one per GPU, held from the first call on that GPU until the
 * process ends.  The call allocates and frees nothing (no hipMalloc, no
 * allocating library routine); it only enqueues the two kernels on `stream`.
 *   - Limit: the workspace pa_decode_step would need for these sizes
 *     (pa_decode_workspace_bytes) must fit PA_NOALLOC_SCRATCH_BYTES, else
 *     PA_ERR_WORKSPACE before any launch.  It is 2 * 256 * ceil(4 (N + 1) / 256)
 *     bytes plus 2 * W * (Hq / Hkv) * (d_head + 4) * 4, W = 4 waves per CU
 *     (1024 on 256 CUs): up to Hq / Hkv = 7 at d_head 128 on MI355X (the 8B
 *     GQA shape, Hq / Hkv = 4, needs 4.3 MB).
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind; no word of it needs clearing (each call writes every word it
 *     reads).  Calls that may overlap in time on one GPU (other streams, other
 *     host threads) race on the array and must be serialised by the caller.
 *   - PA_ERR_HIP when the runtime cannot give the array's device address.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int pa_decode_step_noalloc(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                           void* v_pool, const int32_t* slot_mapping, int32_t* block_tables,
                           int32_t* context_lens, int num_seqs, int Hq, int Hkv, int d_head, int block_size,
                           float scale, int max_blocks_per_seq, int max_context_len, int num_blocks, int dtype,
                           void* stream);

/* pa_decode_shared: pa_decode, with the full blocks that a group of
 * consecutive rows shares read once for the whole group.  A full block
 * referenced by several sequences is immutable, so every sharer sees the same
 * keys and values in it ("PagedAttention: Virtual Memory for the KV Cache",
 * section 15), and a row's attention is the common-maximum merge of the
 * summaries of its shared tokens and of the rest ("PagedAttention in vLLM:
 * scattered memory, exact attention", section 11).  The output is that of
 * pa_decode on the same arguments (same tolerance; not bitwise, as the split
 * differs).
 *
 *   groups      int32 [num_groups][3] = (first row, rows, P tokens),
 *               device-readable (device memory, or pinned host memory
 *               mapped for the device), e.g. from pa_bm_shared_groups.
 *               Rows first .. first + rows - 1 read tokens 0 .. P - 1
 *               through row `first`'s table.
 *   num_groups  >= 0; 0 is plain pa_decode
 *
 * Precondition (caller): for every group, the members' block_tables rows
 * agree on their first P / block_size entries.  Everything else is checked
 * on the device and a group that fails is ignored for this call, which
 * leaves the result exact: rows outside the batch, rows claimed by another
 * group (one of the two is used), P < block_size.  P is cut to the shortest
 * member's context length and rounded down to whole blocks; a group keeps at
 * most 32 / (Hq / Hkv) rows (later rows attend alone).  The groups must stay
 * unchanged until the call has run.  Served by the shared-prefix kernel for
 * bf16, Hq / Hkv <= 16, num_seqs <= 1024, num_groups <= 512; other shapes run
 * pa_decode (the groups unused).  Workspace: pa_decode_shared_workspace_bytes.
 * Other arguments and errors as for pa_decode.
 */
int pa_decode_shared(void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* context_lens, const int32_t* groups,
                     int num_groups, int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                     int max_blocks_per_seq, int max_context_len, int num_blocks, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* pa_decode_step_shared: pa_decode_step with groups as for pa_decode_shared.
 * Each row's new token belongs to its own part, so the rows move forward
 * exactly as with pa_decode_step; the groups stay valid for the next step as
 * long as P stays within every member's table (shared blocks are never
 * written).  Shapes outside the shared-prefix kernel run pa_decode_step;
 * shapes outside pa_decode_step return PA_ERR_UNSUPPORTED. */
int pa_decode_step_shared(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                          void* v_pool, const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                          const int32_t* groups, int num_groups, int num_seqs, int Hq, int Hkv, int d_head,
                          int block_size, float scale, int max_blocks_per_seq, int max_context_len, int num_blocks,
                          int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pa_decode_shared / pa_decode_step_shared need for these
 * sizes on the current device (pa_decode's when the groups go unused). */
size_t pa_decode_shared_workspace_bytes(int num_seqs, int num_groups, int Hq, int Hkv, int d_head, int block_size,
                                        int max_context_len, int dtype);

/* Workspace bytes pa_decode needs for these sizes on the current device
 * (0 when no split is used); dtype PA_FP8_E4M3 or PA_INT8 gives
 * pa_decode_fp8's or pa_decode_int8's (the same size). */
size_t pa_decode_workspace_bytes(int num_seqs, int Hq, int Hkv, int d_head, int block_size,
                                 int max_context_len, int dtype);

/* Tokens per partition that pa_decode uses for these sizes (for reporting);
 * 0 when the balanced persistent kernel is used (bf16, Hq / Hkv <= 16,
 * num_seqs <= 3072), whose split follows equal per-wave tile ranges. */
int pa_decode_partition_tokens(int num_seqs, int Hq, int Hkv, int d_head, int block_size,
                               int max_context_len, int dtype);

/* ---- KV append ---------------------------------------------------------------
 *
 * pa_append_kv: write each new token's key and value, for all KV heads, into
 * its slot: block slot / B, offset slot % B ("PagedAttention: Virtual Memory
 * for the KV Cache", section 16: the appended position is written into its
 * block at its offset).  Bit-exact copy of the input elements.
 *
 *   k_new, v_new   [num_tokens][Hkv][d_head], element type `dtype`
 *   slot_mapping   int32 [num_tokens]; slot < 0 skips the token; slots at or
 *                  beyond num_blocks * block_size are skipped as well
 * Slots must be distinct within one call.
 */
int pa_append_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, int num_tokens, int Hkv, int d_head,
                 int block_size, int num_blocks, int dtype, void* stream);

/* pa_append_step: pa_append_kv for one decode step of a batch whose block
 * tables and lengths stay on the device, which also moves each row forward
 * as the host block manager's append does ("PagedAttention: Virtual Memory
 * for the KV Cache", sections 3 and 16: position S of a sequence lives in
 * logical block S / B at offset S % B).  For row n with slot = slot_mapping[n]
 * and S = context_lens[n] before the call:
 *
 *     K, V of token n written at `slot` (as pa_append_kv)
 *     block_tables[n][S / B] = slot / B;  context_lens[n] = S + 1
 *
 * so the device batch equals what pa_bm_build_batch returns after the same
 * pa_bm_append_slots, without uploading the tables again.
 *
 *   k_new, v_new   [num_seqs][Hkv][d_head], element type `dtype`
 *   slot_mapping   int32 [num_seqs], device; slot < 0 or at or beyond
 *                  num_blocks * block_size skips the row entirely
 *   block_tables   int32 [num_seqs][max_blocks_per_seq], device, updated
 *   context_lens   int32 [num_seqs], device, updated
 * A row whose slot does not sit at its next position (slot % B != S % B,
 * S < 0 or S / B >= max_blocks_per_seq) keeps its table and length; its
 * key and value are still written.  Slots must be distinct within one call.
 */
int pa_append_step(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                   const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                   int num_seqs, int max_blocks_per_seq, int Hkv, int d_head, int block_size,
                   int num_blocks, int dtype, void* stream);

/* ---- copy-on-write block copy ------------------------------------------------
 *
 * pa_copy_blocks: for each pair (src, dst) and each of num_layers layers,
 * copy block src of both pools over block dst, all KV heads and all slots
 * ("PagedAttention: Virtual Memory for the KV Cache", sections 15-16: a shared
 * tail block is cloned before a sequence writes into it).  Bit-exact.
 *
 *   src_dst_pairs  int32 [num_pairs][2] on the device; destinations are
 *                  distinct and no destination is a source in the same call;
 *                  pairs with an id outside [0, num_blocks) are skipped
 *   layer_stride_elems  elements between consecutive layers of each pool
 *                  (ignored when num_layers == 1)
 */
int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_dst_pairs, int num_pairs,
                   int Hkv, int d_head, int block_size, int num_blocks, int num_layers,
                   int64_t layer_stride_elems, int dtype, void* stream);

/* ---- FP8 (E4M3) KV cache ------------------------------------------------------
 *
 * A cache of 8-bit codes halves the bytes per token of a bf16 cache
 * ("PagedAttention and KV Memory", "Alternatives and ecosystem": quantized
 * KV cuts per-token size and combines with paging).  Attention over it is the
 * exact attention over the values the codes stand for ("PagedAttention in
 * vLLM: scattered memory, exact attention", sections 8 and 11: quantization
 * changes precision, not the attention rule).
 *
 * Codes: FP8 E4M3 of the OCP 8-bit floating point format (exponent bias 7,
 * subnormals, no infinities, NaN = 0x7F / 0xFF, largest finite 448).
 * Scales: fp32, one per (physical block, KV head) for keys and one for
 * values, interleaved in one device array `scales` [num_blocks][Hkv][2]
 * owned by the caller, 8-byte aligned (PA_ERR_INVALID_ARG otherwise),
 * positive and finite:
 *
 *     key scale of block pb, KV head j:   scales[(pb * Hkv + j) * 2 + 0]
 *     value scale:                        scales[(pb * Hkv + j) * 2 + 1]
 *
 * so the decode fetches both of a (block, head) with one 8-byte load.  Key
 * code c of block pb, KV head j stands for value(c) * key scale, value codes
 * likewise.  Static per-head scaling is the case where all blocks of a head
 * carry the same scales.
 * Pool layout: as above with E = 1: K and V codes [num_blocks][Hkv][B][D].
 */

/* pa_decode over an FP8 cache.  q and out are bf16 [num_seqs][Hq][d_head];
 * the other arguments, the workspace (pa_decode_workspace_bytes with dtype
 * PA_FP8_E4M3), the split and the errors are as for pa_decode.  Scores are
 * scale * key scale * dot(q, value(codes)) and P.V weighs value(codes) *
 * value scale, accumulated in fp32.  Served for Hq / Hkv <= 16, num_seqs <= 3072,
 * d_head in {64, 128}, block_size in {8, 16, 32}; other shapes return
 * PA_ERR_UNSUPPORTED.  Scales of blocks the tables reach must be positive and
 * finite; a block id outside [0, num_blocks) is never dereferenced. */
int pa_decode_fp8(void* out, const void* q, const void* k_pool, const void* v_pool, const float* scales,
                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                  int Hq, int Hkv, int d_head, int block_size, float scale, int max_blocks_per_seq,
                  int max_context_len, int num_blocks, void* workspace, size_t workspace_bytes, void* stream);

/* pa_append_kv into an FP8 cache: each element x of token t's bf16 key and
 * value (k_new, v_new [num_tokens][Hkv][d_head]) is stored at slot
 * slot_mapping[t] ("PagedAttention: Virtual Memory for the KV Cache",
 * section 16) as the sign of x and the finite E4M3 magnitude nearest to the
 * real quotient |x| / scale of the destination (block, KV head), ties to an
 * even mantissa; magnitudes beyond 448 saturate to 448.  NaN input, or a scale
 * that is not positive and finite, stores 0x7F.  Slots as for pa_append_kv.
 * Deterministic: the codes depend only on x and the scale. */
int pa_append_kv_fp8(void* k_pool, void* v_pool, const float* scales, const void* k_new, const void* v_new, const int32_t* slot_mapping, int num_tokens,
                     int Hkv, int d_head, int block_size, int num_blocks, void* stream);

/* pa_append_step into an FP8 cache: the codes as pa_append_kv_fp8 stores
 * them (row n's token at slot_mapping[n]) and each row moved forward as
 * pa_append_step does (block_tables[n][S / B] = slot / B, context_lens[n] =
 * S + 1 when the slot is the row's next position).  k_new, v_new bf16
 * [num_seqs][Hkv][d_head]; other arguments as for pa_append_step. */
int pa_append_step_fp8(void* k_pool, void* v_pool, const float* scales, const void* k_new,
                       const void* v_new, const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                       int num_seqs, int max_blocks_per_seq, int Hkv, int d_head, int block_size, int num_blocks,
                       void* stream);

/* pa_decode_step over an FP8 cache: one whole decode step of the batch
 * ("PagedAttention: Virtual Memory for the KV Cache", sections 13 and 16).
 * Row n attends to its S cached tokens and to its new token (bf16 k_new /
 * v_new [num_seqs][Hkv][d_head]) as the cache will hold it: the codes
 * pa_append_kv_fp8 stores for it under the scales of the block its slot
 * lies in, slot = slot_mapping[n] (device-readable, as for pa_decode_step).
 * Then those codes are stored and the row moved forward as pa_append_step_fp8
 * does.  Where every slot is its row's next position the codes, tables and
 * lengths are bit for bit those of pa_append_step_fp8, and the output is the
 * attention over the cache that append leaves (the decode kernel attends to
 * the cached tokens, the merge kernel adds the new token as one more piece,
 * so the output bits may differ from pa_append_step_fp8 + pa_decode_fp8
 * within the decode's tolerance).  A row whose slot lies outside
 * [0, num_blocks * block_size)
 * has no block whose scales its codes could use: it attends to its S cached
 * tokens only (S = 0 gives zeros), and its codes, table and length stay.
 * A row whose slot is in the pool but not its next position attends to its
 * new token and keeps its table and length (its codes are not stored).
 * Scales of the blocks the slots lie in must be set before the call.  Other
 * arguments, the workspace (dtype PA_FP8_E4M3), shapes and errors as for
 * pa_decode_fp8 and pa_decode_step. */
int pa_decode_step_fp8(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                       const float* scales, const int32_t* slot_mapping, int32_t* block_tables,
                       int32_t* context_lens, int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                       int max_blocks_per_seq, int max_context_len, int num_blocks, void* workspace,
                       size_t workspace_bytes, void* stream);

/* pa_copy_blocks for an FP8 cache: codes of block src over block dst, and its
 * scales with them, scales[dst][*][*] = scales[src][*][*]
 * ("PagedAttention: Virtual Memory for the KV Cache", sections 15-16).
 * Bit-exact.  layer_stride_elems counts codes (bytes) between layers of each
 * pool, scale_layer_stride floats between layers of the scale array (at least
 * num_blocks * Hkv * 2; both ignored when num_layers == 1).  Pairs as for
 * pa_copy_blocks. */
int pa_copy_blocks_fp8(void* k_pool, void* v_pool, float* scales, const int32_t* src_dst_pairs,
                       int num_pairs, int Hkv, int d_head, int block_size, int num_blocks, int num_layers,
                       int64_t layer_stride_elems, int64_t scale_layer_stride, void* stream);

/* ---- INT8 KV cache -----------------------------------------------------------------
 *
 * The other quantized format that "PagedAttention and KV Memory"
 * ("Alternatives and ecosystem") names beside FP8: the same bytes per token,
 * the same scales and layout as the FP8 cache above, integer codes.  Attention
 * over it is the exact attention over the values the codes stand for
 * ("PagedAttention in vLLM: scattered memory, exact attention", sections 8
 * and 11).
 *
 * Codes: signed 8-bit two's complement integers; code c of block pb, KV head j
 * stands for c * scale[pb][j].  The appenders write only -127..127; a stored
 * -128 stands for -128 * scale.  Scales, pool layout and ownership as for the
 * FP8 cache.
 */

/* pa_decode over an INT8 cache: as pa_decode_fp8 with the values c * scale
 * (workspace: pa_decode_workspace_bytes with dtype PA_INT8; shapes, split and
 * errors as for pa_decode_fp8). */
int pa_decode_int8(void* out, const void* q, const void* k_pool, const void* v_pool, const float* scales,
                   const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                   int Hq, int Hkv, int d_head, int block_size, float scale, int max_blocks_per_seq,
                   int max_context_len, int num_blocks, void* workspace, size_t workspace_bytes, void* stream);

/* pa_append_kv into an INT8 cache: each element x of token t's bf16 key and
 * value is stored at slot slot_mapping[t] ("PagedAttention: Virtual Memory for
 * the KV Cache", section 16) as the integer nearest to the real quotient
 * x / scale of the destination (block, KV head), ties to even, clamped to
 * -127..127.  NaN input, or a scale that is not positive and finite, stores 0
 * (an 8-bit integer has no NaN).  Other arguments as for pa_append_kv_fp8. */
int pa_append_kv_int8(void* k_pool, void* v_pool, const float* scales, const void* k_new, const void* v_new, const int32_t* slot_mapping, int num_tokens,
                      int Hkv, int d_head, int block_size, int num_blocks, void* stream);

/* pa_append_step into an INT8 cache: the codes as pa_append_kv_int8 stores
 * them and each row moved forward as pa_append_step does; arguments as for
 * pa_append_step_fp8. */
int pa_append_step_int8(void* k_pool, void* v_pool, const float* scales, const void* k_new,
                        const void* v_new, const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                        int num_seqs, int max_blocks_per_seq, int Hkv, int d_head, int block_size, int num_blocks,
                        void* stream);

/* pa_decode_step_fp8 over an INT8 cache (workspace: dtype PA_INT8). */
int pa_decode_step_int8(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const float* scales, const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens, int num_seqs, int Hq, int Hkv, int d_head,
                        int block_size, float scale, int max_blocks_per_seq, int max_context_len, int num_blocks,
                        void* workspace, size_t workspace_bytes, void* stream);

/* pa_copy_blocks for an INT8 cache: codes and scales of block src over block
 * dst, exactly as pa_copy_blocks_fp8 (the copy moves bytes and scales,
 * whatever the codes mean). */
int pa_copy_blocks_int8(void* k_pool, void* v_pool, float* scales, const int32_t* src_dst_pairs,
                        int num_pairs, int Hkv, int d_head, int block_size, int num_blocks, int num_layers,
                        int64_t layer_stride_elems, int64_t scale_layer_stride, void* stream);

/* ---- swapping blocks between pools ----------------------------------------------
 *
 * pa_swap_blocks: preemption by swapping ("PagedAttention: Virtual Memory for
 * the KV Cache", section 19) moves whole blocks between the device pool and a
 * host pool.  For each pair (src, dst) of src_dst_pairs (int32 [num_pairs][2],
 * device-readable), block src of the source pools is copied to block dst of
 * the destination pools, K and V, in each of num_layers layers; bit-exact.
 * Both pools have the device pool's per-block layout (see the top of this
 * file); each is device memory or pinned host memory mapped for the device
 * (pass the device pointer of the mapping), so one call moves a batch of
 * scattered blocks over PCIe with no staging.  Use the pairs pa_bm_swap_out
 * (device -> host) or pa_bm_swap_in (host -> device) returns, on the stream
 * that runs the decode, before the released blocks are reused / before the
 * swapped-in sequences are decoded.
 *   src_num_blocks / dst_num_blocks  blocks in one layer of each pool (a pair
 *                     outside them is skipped)
 *   *_layer_stride_elems  elements between layers of each pool (ignored when
 *                     num_layers == 1)
 *   dtype             PA_F32 or PA_BF16; pa_swap_blocks_fp8 moves FP8 codes
 *                     and their per-(block, KV head) key and value scales
 *                     (interleaved [num_blocks][Hkv][2] arrays; scale strides
 *                     in floats, at least blocks * Hkv * 2),
 *                     pa_swap_blocks_int8 INT8 codes and scales the same way.
 * Argument errors as for pa_copy_blocks. */
int pa_swap_blocks(void* dst_k_pool, void* dst_v_pool, const void* src_k_pool, const void* src_v_pool,
                   const int32_t* src_dst_pairs, int num_pairs, int Hkv, int d_head, int block_size, int dtype,
                   int src_num_blocks, int dst_num_blocks, int num_layers, int64_t src_layer_stride_elems,
                   int64_t dst_layer_stride_elems, void* stream);
int pa_swap_blocks_fp8(void* dst_k_pool, void* dst_v_pool, float* dst_scales, const void* src_k_pool,
                       const void* src_v_pool, const float* src_scales, const int32_t* src_dst_pairs, int num_pairs, int Hkv, int d_head,
                       int block_size, int src_num_blocks, int dst_num_blocks, int num_layers,
                       int64_t src_layer_stride_elems, int64_t dst_layer_stride_elems, int64_t src_scale_layer_stride,
                       int64_t dst_scale_layer_stride, void* stream);
int pa_swap_blocks_int8(void* dst_k_pool, void* dst_v_pool, float* dst_scales, const void* src_k_pool,
                        const void* src_v_pool, const float* src_scales, const int32_t* src_dst_pairs, int num_pairs, int Hkv, int d_head,
                        int block_size, int src_num_blocks, int dst_num_blocks, int num_layers,
                        int64_t src_layer_stride_elems, int64_t dst_layer_stride_elems, int64_t src_scale_layer_stride,
                        int64_t dst_scale_layer_stride, void* stream);

/* ---- host block manager ------------------------------------------------------
 *
 * Free list, per-block reference counts, block tables, fork and copy-on-write
 * of a shared unaligned tail ("PagedAttention: Virtual Memory for the KV
 * Cache", sections 14-17 and the teaching allocator of section 20).  Host
 * only; no device calls.  A handle is not thread-safe: one thread at a time.
 *
 * Rules:
 *   - a sequence of S tokens holds ceil(S / B) blocks;
 *   - fork copies the parent's table and adds one reference to every block;
 *   - appending at position S: if S % B == 0 a fresh block is taken; else if
 *     the tail block is shared (ref > 1) a fresh block is taken, the pair
 *     (old tail, fresh block) is reported for a device block copy, the old
 *     tail loses one reference and the table points at the fresh block; else
 *     the token is written in place.  The returned slot is always in a block
 *     with exactly one reference;
 *   - release drops one reference per block; blocks reaching zero return to
 *     the free list, which is LIFO (the last block released is handed out
 *     next).  The caller must not let later work reuse a freed block before
 *     earlier device work that reads it is ordered before it (same stream);
 *   - any failure (PA_ERR_*) leaves the manager exactly as it was.
 */
typedef struct pa_bm pa_bm;

typedef struct pa_bm_stats_t {
  int64_t num_blocks;       /* pool size                                          */
  int64_t num_free;         /* blocks on the free list                            */
  int64_t num_used;         /* blocks with at least one reference                 */
  int64_t num_seqs;         /* live sequences                                     */
  int64_t cow_copies;       /* copy-on-write pairs issued so far                  */
  int64_t stored_tokens;    /* valid token slots in used blocks, shared ones once */
  int64_t tail_waste_slots; /* num_used * block_size - stored_tokens              */
} pa_bm_stats_t;

/* Create a manager of num_blocks blocks of block_size tokens.  pop_order
 * (nullable, host, num_blocks distinct ids) fixes the order in which free
 * blocks are first handed out; NULL hands out 0, 1, 2, ...  Returns NULL on
 * invalid sizes or a pop_order that is not a permutation. */
pa_bm* pa_bm_create(int num_blocks, int block_size, const int32_t* pop_order);
void pa_bm_destroy(pa_bm* bm);

/* New sequence of num_tokens >= 1 tokens (its prompt): ceil(n / B) blocks. */
int pa_bm_add_seq(pa_bm* bm, int64_t seq, int num_tokens);

/* New sequence `child` sharing every block of `parent`. */
int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);

/* Reserve the slot of the next position of `seq`.  *slot receives
 * block * B + offset; *cow_src / *cow_dst receive the copy-on-write pair or
 * -1 / -1.  On failure all three receive -1. */
int pa_bm_append_slot(pa_bm* bm, int64_t seq, int32_t* slot, int32_t* cow_src, int32_t* cow_dst);

/* Batch append, all-or-nothing, in array order: slots[i] for seqs[i];
 * cow_pairs (capacity n pairs, int32 [n][2]) receives the copy-on-write pairs
 * in order and *num_pairs their count.  On failure nothing changes and
 * *num_pairs receives -(index of the failing sequence) - 1. */
int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, int n, int32_t* slots,
                       int32_t* cow_pairs, int* num_pairs);

/* Release a sequence. */
int pa_bm_free_seq(pa_bm* bm, int64_t seq);

/* Fill block_tables_out int32 [n][max_blocks_per_seq] (unused entries 0) and
 * context_lens_out int32 [n] for the listed sequences. */
int pa_bm_build_batch(pa_bm* bm, const int64_t* seqs, int n, int max_blocks_per_seq,
                      int32_t* block_tables_out, int32_t* context_lens_out);

/* Groups of consecutive batch rows that read the same full leading blocks,
 * for pa_decode_shared.  A full block referenced by several sequences is
 * immutable and may be read by all of them at once ("PagedAttention: Virtual
 * Memory for the KV Cache", section 15), so a decode can read it once for the
 * whole group.  Row i is seqs[i]; row i holds floor(len / B) full blocks.
 * Rows are walked in order: a run starts at a row with L = its full-block
 * count; the next row joins while the run has fewer than max_members rows,
 * the row's table starts with c >= 1 of the run's first L entries (among the
 * row's own full blocks) and k * c >= (k - 1) * L for the k rows so far (the
 * bytes the run saves do not drop); L becomes c.  Every run of >= 2 rows
 * with L >= 1 is written to groups_out as int32 [3] = (first row, rows,
 * L * B shared tokens), in row order; *num_groups receives their count.
 *   groups_out   host int32 [cap][3], caller-owned (nullable when cap == 0)
 * Errors: PA_ERR_NOT_FOUND for an unknown sequence; PA_ERR_INVALID_ARG for
 * bad arguments or when more than cap groups are found (*num_groups then
 * holds the number needed).  Nothing in the manager changes. */
int pa_bm_shared_groups(pa_bm* bm, const int64_t* seqs, int n, int max_members, int32_t* groups_out, int cap,
                        int* num_groups);

/* ---- prefix cache ------------------------------------------------------------
 *
 * Automatic prefix caching ("PagedAttention: Virtual Memory for the KV
 * Cache", sections 18-19; "PagedAttention in vLLM: scattered memory, exact
 * attention", section 6; "PagedAttention and KV Memory", "Prefix caching"):
 * a full block is identified by its token ids together with every token
 * before it in its sequence, so equal text after a different prefix never
 * matches.  A cached block whose reference count drops to 0 is kept (idle)
 * and reused by a later request whose prefix matches (0 -> 1); under
 * pressure an allocation reclaims the least recently released idle block
 * before it fails.  Host only.
 *
 *   - only full blocks are cached: a prompt's full blocks, and a block that
 *     fills up through pa_bm_append_tokens with known token ids; a block
 *     whose chain is cached already stays uncached;
 *   - a lookup takes the longest run of leading full blocks whose chains are
 *     cached and stops at the first miss;
 *   - appends without token ids (pa_bm_append_slot(s)), and sequences added
 *     with pa_bm_add_seq, end a sequence's chain: its later blocks are not
 *     cached;
 *   - release walks a sequence's table from its last block to its first; a
 *     cached block reaching 0 becomes the most recently released idle block,
 *     any other block goes to the free list; allocation takes the free list
 *     first, then evicts the least recently released idle block;
 *   - a match compares the block's token ids and a 64-bit hash of the tokens
 *     before it: a false match needs a 64-bit collision of two different
 *     prefixes that end in the same block of tokens;
 *   - batch appends check capacity first (a dry run of the copy-on-write
 *     decisions) and then cannot fail.
 *
 * A reused block's KV is whatever its first owner's prefill wrote: that
 * prefill must be ordered before the decode that reads it (one stream). */
typedef struct pa_bm_cache_stats_t {
  int64_t enabled;     /* 1 once pa_bm_enable_prefix_cache succeeded          */
  int64_t num_cached;  /* blocks holding a cached chain (in use or idle)     */
  int64_t num_idle;    /* cached blocks without references (evictable)       */
  int64_t hit_blocks;  /* blocks reused by pa_bm_add_seq_tokens so far       */
  int64_t evictions;   /* idle blocks reclaimed by allocations so far        */
} pa_bm_cache_stats_t;

/* Turn the prefix cache on.  Only while the manager holds no sequence
 * (PA_ERR_INVALID_ARG otherwise); it stays on. */
int pa_bm_enable_prefix_cache(pa_bm* bm);

/* New sequence with prompt token ids tokens[0 .. num_tokens - 1] (host,
 * caller-owned).  Reuses the longest cached run of its leading full blocks
 * and takes fresh blocks for the rest; *cached_tokens (nullable) receives the
 * number of leading tokens whose KV is already there (a multiple of B), which
 * the caller's prefill may skip.  All-or-nothing (PA_ERR_NO_FREE_BLOCKS leaves
 * the manager unchanged).  Without the prefix cache: pa_bm_add_seq. */
int pa_bm_add_seq_tokens(pa_bm* bm, int64_t seq, const int32_t* tokens, int num_tokens, int* cached_tokens);

/* pa_bm_append_slots, with the appended tokens' ids (tokens[i] for seqs[i];
 * NULL: unknown), so blocks that fill up can be cached. */
int pa_bm_append_tokens(pa_bm* bm, const int64_t* seqs, const int32_t* tokens, int n, int32_t* slots,
                        int32_t* cow_pairs, int* num_pairs);

/* Prefix-cache counters. */
int pa_bm_cache_stats(pa_bm* bm, pa_bm_cache_stats_t* out);

/* Copy the idle cached blocks, least recently released first (the eviction
 * order); *n_out = their number. */
int pa_bm_idle_list(pa_bm* bm, int32_t* out, int cap, int* n_out);

/* ---- swapping ------------------------------------------------------------------
 *
 * Preemption by swapping ("PagedAttention: Virtual Memory for the KV Cache",
 * section 19): a running sequence's blocks move to host memory, its device
 * blocks serve other requests, and it comes back once device blocks are
 * released.  The manager tracks a pool of host blocks (ids 0 .. H - 1, in a
 * host pool the caller allocates with the device pool's per-block layout);
 * the data moves with pa_swap_blocks.  Host only.
 *
 *   - pa_bm_swap_out moves the listed resident sequences: each distinct
 *     device block they reference (in order of first appearance: sequence
 *     order, then table order) gets one host block that takes over their
 *     references; a block also referenced by a sequence outside the list
 *     keeps those references (the host copy belongs to the listed
 *     sequences), any other block is released (to the free list, or the idle
 *     cache if it is cached).  Their tables then hold host ids.
 *     pairs_out receives (device block, host block) per distinct block: copy
 *     them device -> host before any later work reuses the released blocks.
 *   - pa_bm_swap_in brings the listed swapped sequences back into fresh
 *     device blocks (may evict idle cached blocks); pairs_out receives
 *     (host block, device block): copy them host -> device before the
 *     sequences are decoded.  Sharing among the listed sequences is kept.
 *   - both are all-or-nothing; a sequence listed twice, or in the wrong state,
 *     is PA_ERR_INVALID_ARG; more pairs than cap is PA_ERR_INVALID_ARG with
 *     *num_pairs = the number needed; nothing changes on any error.
 *   - a swapped sequence cannot be appended to, forked, batched or grouped
 *     (PA_ERR_INVALID_ARG); pa_bm_free_seq returns its host blocks;
 *     pa_bm_block_table returns its host ids.
 */

/* A host pool of num_host_blocks blocks (once).  pop_order (nullable, host)
 * fixes the hand-out order as in pa_bm_create. */
int pa_bm_enable_host_pool(pa_bm* bm, int num_host_blocks, const int32_t* pop_order);
int pa_bm_swap_out(pa_bm* bm, const int64_t* seqs, int n, int32_t* pairs_out, int cap, int* num_pairs);
int pa_bm_swap_in(pa_bm* bm, const int64_t* seqs, int n, int32_t* pairs_out, int cap, int* num_pairs);
/* Swapped sequences, free host blocks, host blocks in the pool. */
int pa_bm_swap_stats(pa_bm* bm, int64_t* num_swapped, int64_t* host_free, int64_t* host_blocks);

/* Reference count of a block (-1 for an id outside the pool). */
int pa_bm_refcount(pa_bm* bm, int block);
/* Number of blocks on the free list (idle cached blocks not included). */
int pa_bm_num_free(pa_bm* bm);
/* Length of a sequence in tokens (-1 if unknown). */
int64_t pa_bm_seq_len(pa_bm* bm, int64_t seq);
/* Copy a sequence's table into out (capacity cap); *n_out = its length. */
int pa_bm_block_table(pa_bm* bm, int64_t seq, int32_t* out, int cap, int* n_out);
/* Copy the free list in hand-out order (next block first). */
int pa_bm_free_list(pa_bm* bm, int32_t* out, int cap, int* n_out);
/* True (1) when a new sequence of num_tokens tokens fits the free blocks
 * (and the idle cached blocks, which an allocation may reclaim). */
int pa_bm_can_allocate(pa_bm* bm, int num_tokens);
/* Pool accounting in the terms of the first page's section 17. */
int pa_bm_stats(pa_bm* bm, pa_bm_stats_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

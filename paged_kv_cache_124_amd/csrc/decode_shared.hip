// Paged decode attention, bf16, with full blocks shared by a group of
// sequences read once for the whole group.
//
// Why it is exact ("PagedAttention: Virtual Memory for the KV Cache", section
// 15; "PagedAttention in vLLM: scattered memory, exact attention", section
// 11): a full block referenced by several sequences is immutable, so every
// sharer sees the same keys and values in it.  The online softmax of a row
// may take its tokens in any grouping, so when rows first .. first + count - 1
// of the batch hold the same physical blocks for their first P / B table
// entries, one pass over those blocks can serve all of them at once, with
// every member's queries as columns of the same matrix-core products, and
// each member's remaining tokens can follow in the same pass with only that
// member's columns taking part.
//
// Work decomposition (the persistent equal split of decode_stream.hip over
// "units" instead of sequences):
//   unit n < N       sequence n without a group: its tokens, 32 per tile;
//                    a sequence in a group has no tiles of its own;
//   unit N + i       group i: ceil(P_i / 32) prefix tiles read through the
//                    table row of its first member with count_i * G query
//                    columns (member m, head h -> column m G + h; at most 32),
//                    then each member's own tokens P_i .. S + new, 32 per tile
//                    through the member's row, the other members' columns
//                    masked out (their scores -inf: no weight, no change).
// Tiles of all (unit, KV head) segments form one list; wave w takes tiles
// [w T / W, (w + 1) T / W).  A group tile is one 16 KiB read of keys and
// values used by two 16-column blocks of matrix-core products instead of one.
// A segment a wave finishes whole is written directly (a group's for all its
// rows); a segment cut by range boundaries leaves an (m, z, u) record per
// piece and column (32 rows per wave slot), which `merge_shared` combines
// per (sequence, KV head) in wave order.
//
// Groups that are not usable are ignored, which keeps the result exact: a
// group is used only when all its rows lie in the batch, no other group
// claims one of them and it shares at least one whole block; its P is cut to
// the shortest member's cached length, rounded down to whole blocks, and its
// rows to 32 / G (members past that compute alone).  The caller guarantees
// what the kernel cannot see: the members' table rows agree on the first
// P / B entries.

#include <cstdlib>

#include "common.h"
#include "decode_stream.h"
#include "decode_tile.h"

namespace pa {
namespace {

constexpr int kShMaxSeqs = 1024;
constexpr int kShMaxGroups = 512;
constexpr int kShCols = 32;  // query columns of one tile: two 16-column blocks

// LDS of the kernel besides the stages: lengths and prefix sums of the units,
// the group of each sequence, and per group its first row, rows, shared
// tokens and tiles.
size_t shared_lds(int n, int g) { return (3 * static_cast<size_t>(n) + 6 * static_cast<size_t>(g) + 1) * 4; }

// Position in the tile list: unit n, KV head j, tile ti of the segment; for a
// group unit's member tiles also the member m and its tile k (m = -1 for
// every other tile).
struct UTile {
  int n, j, ti, m, k;
};

// Wave-uniform views of the unit tables in LDS.
struct Units {
  const int32_t* s_len;    // [units] packed tokens: group units P << 2; sequences as in decode_stream,
                           // counted from P for a sequence in a group
  const int32_t* s_pre;    // [units + 1]
  const int32_t* s_gid;    // [N]
  const int32_t* s_gfirst; // [groups]
  const int32_t* s_gcount;
  const int32_t* s_gtok;
  int n_seqs, g, hkv;
  __device__ bool is_group(int u) const { return u >= n_seqs; }
  __device__ int tiles(int u) const { return s_pre[u + 1] - s_pre[u]; }
  __device__ int prefix_tiles(int u) const { return (s_gtok[u - n_seqs] + 31) >> 5; }
  // tiles of member m's own tokens in group unit u
  __device__ int member_tiles(int u, int m) const {
    return (attended_tokens(s_len[s_gfirst[u - n_seqs] + m]) + 31) >> 5;
  }
  // the first member at or after m with tiles of its own (the last member at most)
  __device__ int next_member(int u, int m) const {
    const int last = s_gcount[u - n_seqs] - 1;
    while (m < last && member_tiles(u, m) == 0) ++m;
    return m;
  }
  // the sequence whose table row, tokens and new token a tile uses
  __device__ int seq_of(const UTile& t) const {
    if (!is_group(t.n)) return t.n;
    return s_gfirst[t.n - n_seqs] + (t.m >= 0 ? t.m : 0);
  }
  // tokens before the tile's token 0 (a multiple of B) and its packed tokens
  __device__ int base(const UTile& t) const { return t.m >= 0 ? s_gtok[t.n - n_seqs] : 0; }
  __device__ int packed(const UTile& t) const { return t.m >= 0 ? s_len[seq_of(t)] : s_len[t.n]; }
  __device__ int t0(const UTile& t) const { return 32 * (t.m >= 0 ? t.k : t.ti); }
  __device__ int cols(int u) const { return is_group(u) ? s_gcount[u - n_seqs] * g : g; }
  // the tile that ends the attended tokens of its sequence (where the new token is)
  __device__ bool ends_seq(const UTile& t) const {
    return t.m >= 0 ? t.k == member_tiles(t.n, t.m) - 1 : (!is_group(t.n) && t.ti == tiles(t.n) - 1);
  }
  __device__ UTile locate(int u, int64_t rem) const {
    UTile t;
    t.n = u;
    const int nt = tiles(u);
    t.j = static_cast<int>(rem / nt);
    t.ti = static_cast<int>(rem - static_cast<int64_t>(t.j) * nt);
    t.m = -1;
    t.k = 0;
    if (is_group(u) && t.ti >= prefix_tiles(u)) {
      int r = t.ti - prefix_tiles(u);
      int m = next_member(u, 0);
      while (r >= member_tiles(u, m) && m < s_gcount[u - n_seqs] - 1) {
        r -= member_tiles(u, m);
        m = next_member(u, m + 1);
      }
      t.m = m;
      t.k = r;
    }
    return t;
  }
};

// What a step needs to know about one tile of the list.  Each lane works out
// the tile of one position of a window of 64 consecutive tiles from the unit
// tables in LDS (a binary search and a walk over the members); a step reads
// its tiles' fields from their lanes (readlane, wave-uniform results).  So no
// LDS lookup lies between one tile's copies and the next's: a new window is
// built once per 62 tiles.
struct TileInfo {
  int n, j, ti, m;   // unit, KV head, tile of the segment, member (-1: not a member's own tile)
  int seq;           // the row whose table, tokens and new token the tile uses
  int packed;        // that row's packed tokens (a group prefix: P << 2), as Units::packed
  int t0, base;      // first token of the tile after base (Units::t0, Units::base)
  int nt;            // tiles of the unit's segment
  int first, count;  // a group's first row and members; a sequence: itself and 1
  int ends;          // the tile ends its row's attended tokens (where the new token is)
};

__device__ __forceinline__ TileInfo tile_info(const Units& us, int n_units, int64_t x) {
  int lo = 0, hi = n_units - 1;
  while (lo < hi) {  // last unit u with hkv * s_pre[u] <= x
    const int mid = (lo + hi + 1) >> 1;
    if (static_cast<int64_t>(us.hkv) * us.s_pre[mid] <= x) lo = mid; else hi = mid - 1;
  }
  const UTile t = us.locate(lo, x - static_cast<int64_t>(us.hkv) * us.s_pre[lo]);
  const bool grp = us.is_group(t.n);
  TileInfo d;
  d.n = t.n;
  d.j = t.j;
  d.ti = t.ti;
  d.m = t.m;
  d.seq = us.seq_of(t);
  d.packed = us.packed(t);
  d.t0 = us.t0(t);
  d.base = us.base(t);
  d.nt = us.tiles(t.n);
  d.first = grp ? us.s_gfirst[t.n - us.n_seqs] : t.n;
  d.count = grp ? us.s_gcount[t.n - us.n_seqs] : 1;
  d.ends = us.ends_seq(t) ? 1 : 0;
  return d;
}

// The tile a lane of the window holds (idx wave-uniform).
__device__ __forceinline__ TileInfo lane_tile(const TileInfo& d, int idx) {
  TileInfo t;
  t.n = __builtin_amdgcn_readlane(d.n, idx);
  t.j = __builtin_amdgcn_readlane(d.j, idx);
  t.ti = __builtin_amdgcn_readlane(d.ti, idx);
  t.m = __builtin_amdgcn_readlane(d.m, idx);
  t.seq = __builtin_amdgcn_readlane(d.seq, idx);
  t.packed = __builtin_amdgcn_readlane(d.packed, idx);
  t.t0 = __builtin_amdgcn_readlane(d.t0, idx);
  t.base = __builtin_amdgcn_readlane(d.base, idx);
  t.nt = __builtin_amdgcn_readlane(d.nt, idx);
  t.first = __builtin_amdgcn_readlane(d.first, idx);
  t.count = __builtin_amdgcn_readlane(d.count, idx);
  t.ends = __builtin_amdgcn_readlane(d.ends, idx);
  return t;
}

// Table entries of a tile: tokens base + t0 .. + 31 of its sequence's row (a
// group's prefix: its first member's), -1 past the tokens in the pool.
template <int B>
__device__ __forceinline__ Tb<32 / B> load_tb_unit(const TileInfo& t, const int32_t* __restrict__ block_tables,
                                                   int max_blocks) {
  const int32_t* row = block_tables + static_cast<int64_t>(t.seq) * max_blocks;
  const int S = pool_tokens(t.packed);
  const int t0 = t.t0;
  const int b0 = (t.base + t0) / B;
  Tb<32 / B> tb;
#pragma unroll
  for (int i = 0; i < 32 / B; ++i) {
    const int e = row[min(b0 + i, max_blocks - 1)];
    tb.blk[i] = t0 + i * B < S ? e : -1;
  }
  return tb;
}

// Rows of q the lane's two columns read for a segment: column c = 16 cb + r
// is head c of a sequence unit (c < G), or member c / G, head c % G of a
// group; padding columns read a valid row whose results are never used.
// Reads LDS only (see the step: no LDS read may follow the next tile's copies).
struct QRows {
  const uint16_t* p[2];
};

template <int D>
__device__ __forceinline__ QRows q_rows(const TileInfo& t, int n_seqs, int g, const uint16_t* __restrict__ q, int hq,
                                        const int (&col_m)[2], const int (&col_h)[2], int r, int gq) {
  QRows qr;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    int seq, h;
    if (t.n < n_seqs) {
      const int c = 16 * cb + r;
      seq = t.n;
      h = c < g ? c : 0;
    } else {
      const bool ok = col_m[cb] < t.count;
      seq = t.first + (ok ? col_m[cb] : 0);
      h = ok ? col_h[cb] : 0;
    }
    qr.p[cb] = q + (static_cast<int64_t>(seq) * hq + t.j * g + h) * D + gq * 8;
  }
  return qr;
}

// Q^T operands of both column blocks (global loads only).
template <int D>
__device__ __forceinline__ void load_q_rows(QOp<D> (&qo)[2], const QRows& qr) {
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int jj = 0; jj < D / 32; ++jj)
      qo[cb].q[jj] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qr.p[cb] + 32 * jj));
}

// One element of a per-column-block array, as an array of one (for
// tile_group<D, 1>); indices stay compile-time, so nothing moves to scratch.
template <typename T>
__device__ __forceinline__ T (&one(T& x))[1] {
  return *reinterpret_cast<T(*)[1]>(&x);
}
template <typename T>
__device__ __forceinline__ const T (&one(const T& x))[1] {
  return *reinterpret_cast<const T(*)[1]>(&x);
}

// A group tile on NC column blocks, all in one pass: the score products, the
// online-softmax updates and the P.V products of the blocks are independent,
// so their latencies overlap (one wave per SIMD has no other wave to hide
// them behind).  Column c takes part when live[cb] (its lane's column); a
// column that does not gets score -inf for every token: no weight, and its
// running state is unchanged.  Same arithmetic as qk_tile + pv_tile per column
// block otherwise; a column whose running maximum is still -inf is kept at
// zero instead of 0 * inf.
template <int D, int NC>
__device__ __forceinline__ void tile_group(Acc<D> (&st)[NC], const Buf<D>& b, const QOp<D> (&qo)[NC], int t0, int S,
                                           bool full, const bool (&live)[NC], float scale_log2, int gq) {
  f32x4 s[NC][2];  // [column block][slab]
#pragma unroll
  for (int cb = 0; cb < NC; ++cb)
#pragma unroll
    for (int a = 0; a < 2; ++a) s[cb][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < D / 32; ++jj)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int cb = 0; cb < NC; ++cb)
        s[cb][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.k[a][jj], qo[cb].q[jj], s[cb][a], 0, 0, 0);
  int n0 = 4, n1 = 4;
  if (!full) {
    n0 = b.blk0 ? min(max(S - (t0 + 4 * gq), 0), 4) : 0;
    n1 = b.blk1 ? min(max(S - (t0 + 16 + 4 * gq), 0), 4) : 0;
  }
  float x[NC][2][4];
  float tmax[NC];
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    tmax[cb] = -INFINITY;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[cb][a][i] = live[cb] && i < (a ? n1 : n0) ? s[cb][a][i] * scale_log2 : -INFINITY;
        tmax[cb] = fmaxf(tmax[cb], x[cb][a][i]);
      }
  }
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) tmax[cb] = max_across_groups(tmax[cb]);
  float alpha[NC];
  bf16x8 phi[NC], plo[NC];
  bool moved = false;
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    const float m_new = fmaxf(st[cb].m, tmax[cb]);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // no token yet: exponents of -inf give 0
    alpha[cb] = __builtin_amdgcn_exp2f(st[cb].m - m_ref);
    st[cb].m = m_new;
    float psum = 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[cb][a][i] - m_ref);
        psum += p;
        const __bf16 h = static_cast<__bf16>(p);
        phi[cb][4 * a + i] = h;
        plo[cb][4 * a + i] = static_cast<__bf16>(p - static_cast<float>(h));
      }
    st[cb].z = st[cb].z * alpha[cb] + psum;
    moved = moved || alpha[cb] != 1.f;
  }
  if (__any(moved)) {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
#pragma unroll
      for (int mm = 0; mm < D / 16; ++mm) st[cb].o[mm] *= alpha[cb];
  }
  uint32_t m0a = 0xffffffffu, m0b = 0xffffffffu, m1a = 0xffffffffu, m1b = 0xffffffffu;
  if (!full) {  // zero values of missing tokens (0 * NaN is NaN)
    m0a = n0 >= 2 ? 0xffffffffu : (n0 == 1 ? 0x0000ffffu : 0u);
    m0b = n0 >= 4 ? 0xffffffffu : (n0 == 3 ? 0x0000ffffu : 0u);
    m1a = n1 >= 2 ? 0xffffffffu : (n1 == 1 ? 0x0000ffffu : 0u);
    m1b = n1 >= 4 ? 0xffffffffu : (n1 == 3 ? 0x0000ffffu : 0u);
  }
#pragma unroll
  for (int mm = 0; mm < D / 16; ++mm) {
    const uint4 w = make_uint4(b.v0[mm].x & m0a, b.v0[mm].y & m0b, b.v1[mm].x & m1a, b.v1[mm].y & m1b);
    const bf16x8 vop = __builtin_bit_cast(bf16x8, w);
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
      st[cb].o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi[cb], st[cb].o[mm], 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
      st[cb].o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo[cb], st[cb].o[mm], 0, 0, 0);
  }
}

// End of a piece of segment t: the normalised outputs (whole segment) or a
// wave-slot record per column.
// `cols` and `first` (the group's first row, or the sequence) are the
// segment's.
template <int D>
__device__ __forceinline__ void flush_unit(Acc<D> (&st)[2], const TileInfo& t, int n_seqs, int g, int cols, int first,
                                           bool whole, int slot, int64_t wave_id, uint16_t* out, float* rec, int hq,
                                           int r, int gq, const int (&col_m)[2], const int (&col_h)[2]) {
  const bool grp = t.n >= n_seqs;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    if (cb == 1 && cols <= 16) break;
    const float zt = sum_across_groups(st[cb].z);
    const int c = 16 * cb + r;
    if (c < cols) {
      if (whole) {
        const float inv = zt > 0.f ? 1.f / zt : 0.f;  // every token left out (blocks outside the pool): zeros
        const int seq = grp ? first + col_m[cb] : t.n;
        const int h = grp ? col_h[cb] : c;
        uint16_t* o = out + (static_cast<int64_t>(seq) * hq + t.j * g + h) * D + 4 * gq;
#pragma unroll
        for (int mm = 0; mm < D / 16; ++mm) {
          const uint32_t lo =
              f32_to_bf16_bits(st[cb].o[mm][0] * inv) | (uint32_t(f32_to_bf16_bits(st[cb].o[mm][1] * inv)) << 16);
          const uint32_t hi =
              f32_to_bf16_bits(st[cb].o[mm][2] * inv) | (uint32_t(f32_to_bf16_bits(st[cb].o[mm][3] * inv)) << 16);
          *reinterpret_cast<uint2*>(o + 16 * mm) = make_uint2(lo, hi);
        }
      } else {
        float* rr = rec + (static_cast<int64_t>(wave_id * 2 + slot) * kShCols + c) * (D + 4);
#pragma unroll
        for (int mm = 0; mm < D / 16; ++mm) *reinterpret_cast<f32x4*>(rr + 4 + 16 * mm + 4 * gq) = st[cb].o[mm];
        if (gq == 0) {
          rr[0] = st[cb].m;
          rr[1] = zt;
        }
      }
    }
  }
  reset(st[0]);
  reset(st[1]);
}

template <int D, int B>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void decode_shared(
    const uint16_t* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ groups, int n_groups, uint16_t* __restrict__ out, float* __restrict__ rec,
    int32_t* __restrict__ seq_info_out, int n_seqs, int hq, int hkv, int g, int max_blocks, int num_blocks,
    float scale_log2, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int32_t* __restrict__ slots_out) {
  const int n_units = n_seqs + n_groups;
  extern __shared__ int32_t sm[];
  int32_t* s_len = sm;                   // [units]
  int32_t* s_pre = s_len + n_units;      // [units + 1] tile prefix sums
  int32_t* s_gid = s_pre + n_units + 1;  // [N] claiming group, then the row's group or -1
  int32_t* s_gfirst = s_gid + n_seqs;    // [groups]
  int32_t* s_gcount = s_gfirst + n_groups;
  int32_t* s_gtok = s_gcount + n_groups;
  int32_t* s_gtiles = s_gtok + n_groups;
  __shared__ int32_t s_wsum[kSW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int gq = lane >> 4;
  const int s_cap = max_blocks * B;
  const int max_members = kShCols / g;
  const int hn = k_new != nullptr ? 1 : 0;  // the step: every row attends to its new token

  // ---- groups: sanitize, claim rows, validate --------------------------------
  for (int i = tid; i < n_seqs; i += 256) s_gid[i] = -1;
  for (int i = tid; i < n_groups; i += 256) {
    const int first = groups[3 * i], cnt = groups[3 * i + 1], tok = groups[3 * i + 2];
    const bool ok = first >= 0 && first < n_seqs && cnt >= 1 && tok >= B;
    s_gfirst[i] = ok ? first : 0;
    s_gcount[i] = ok ? min(min(cnt, n_seqs - first), max_members) : 0;
    s_gtok[i] = ok ? min(tok, s_cap) : 0;
  }
  __syncthreads();
  for (int i = tid; i < n_groups; i += 256)
    for (int m = 0; m < s_gcount[i]; ++m) atomicCAS(&s_gid[s_gfirst[i] + m], -1, i);
  __syncthreads();
  for (int i = tid; i < n_groups; i += 256) {
    const int cnt = s_gcount[i];
    bool ok = cnt >= 1;
    int P = s_gtok[i];
    for (int m = 0; m < cnt; ++m) {
      const int n = s_gfirst[i] + m;
      ok = ok && s_gid[n] == i;
      P = min(P, min(max(context_lens[n], 0), s_cap));  // no member attends past its own tokens
    }
    P -= P % B;
    if (!ok || P < B) P = 0;
    int tiles = (P + 31) >> 5;
    for (int m = 0; m < (P > 0 ? cnt : 0); ++m) {  // each member's own tokens P .. S + new
      const int S = min(max(context_lens[s_gfirst[i] + m], 0), s_cap);
      tiles += (S + hn - P + 31) >> 5;
    }
    s_gtok[i] = P;
    s_gtiles[i] = P > 0 ? tiles : 0;
  }
  __syncthreads();
  for (int i = tid; i < n_groups; i += 256)
    if (s_gtok[i] == 0) s_gcount[i] = 0;
  for (int n = tid; n < n_seqs; n += 256) {  // each thread rewrites its own rows only
    const int i = s_gid[n];
    s_gid[n] = i >= 0 && s_gtok[i] > 0 ? i : -1;
  }
  __syncthreads();

  // ---- tiles per unit and their prefix sums (block-wide scan) ----------------
  int carry = 0;
  for (int base = 0; base < n_units; base += 256) {
    const int u = base + tid;
    int v = 0, packed = 0;
    if (u < n_seqs) {
      const int S_raw = context_lens[u];
      const int S = min(max(S_raw, 0), s_cap);
      const int fits = S_raw >= 0 && S_raw < s_cap ? 1 : 0;
      const int i = s_gid[u];
      const int rel = S + hn - (i >= 0 ? s_gtok[i] : 0);
      v = i >= 0 ? 0 : (rel + 31) >> 5;  // a group member's tiles belong to its group
      packed = (rel << 2) | (fits << 1) | hn;
    } else if (u < n_units) {
      v = s_gtiles[u - n_seqs];
      packed = s_gtok[u - n_seqs] << 2;
    }
#pragma unroll
    for (int dlt = 1; dlt < 64; dlt <<= 1) {
      const int w2 = __shfl_up(v, dlt);
      if (lane >= dlt) v += w2;
    }
    if (lane == 63) s_wsum[wave] = v;
    if (u < n_units) s_len[u] = packed;
    __syncthreads();
    int off = carry;
    for (int w2 = 0; w2 < wave; ++w2) off += s_wsum[w2];
    if (u < n_units) s_pre[u + 1] = off + v;
    carry += s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
  }
  if (tid == 0) s_pre[0] = 0;
  __syncthreads();
  // for the merge kernel, 4 words per row: the first tile and tile count of the
  // unit holding its tokens, the row's first record row there, all units' tiles
  if (blockIdx.x == 0)
    for (int n = tid; n < n_seqs; n += 256) {
      const int i = s_gid[n];
      const int u = i >= 0 ? n_seqs + i : n;
      *reinterpret_cast<int4*>(seq_info_out + 4 * static_cast<int64_t>(n)) =
          make_int4(s_pre[u], s_pre[u + 1] - s_pre[u], i >= 0 ? (n - s_gfirst[i]) * g : 0, s_pre[n_units]);
    }
  // no barrier below this point: waves run independently

  const Units us{s_len, s_pre, s_gid, s_gfirst, s_gcount, s_gtok, n_seqs, g, hkv};
  Split sp;
  sp.init(static_cast<int64_t>(hkv) * s_pre[n_units], static_cast<int64_t>(gridDim.x) * kSW);
  // XCD-major numbering, as in decode_stream
  const int64_t wg = gridDim.x % 8 == 0 ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : blockIdx.x;
  const int64_t wave_id = wg * kSW + wave;
  const int64_t x0 = sp.start(wave_id);
  const int64_t x1 = sp.start(wave_id + 1);
  if (x0 >= x1) return;

  // the window of tiles xb .. xb + 63 (past the range: its last tile again)
  int64_t xb = x0;
  TileInfo mine = tile_info(us, n_units, min(xb + lane, x1 - 1));
  TileInfo cur = lane_tile(mine, 0);
  int piece_start = cur.ti;
  bool first_piece = true;

  int col_m[2], col_h[2];  // member and head of the lane's column in a group tile
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    col_m[cb] = (16 * cb + r) / g;
    col_h[cb] = (16 * cb + r) - col_m[cb] * g;
  }

  Acc<D> st[2];
  reset(st[0]);
  reset(st[1]);
  // The queries of a segment are the same for all its tiles: one set of Q
  // operands, loaded when a segment starts (registers are short here: two
  // column blocks of accumulators, scores and operands).
  QOp<D> qc[2];
  TileInfo nxt = lane_tile(mine, 1);  // the range's last tile again when it has one tile
  Tb<32 / B> tbA = load_tb_unit<B>(cur, block_tables, max_blocks);
  Tb<32 / B> tbB = load_tb_unit<B>(nxt, block_tables, max_blocks);
  load_q_rows<D>(qc, q_rows<D>(cur, n_seqs, g, q, hq, col_m, col_h, r, gq));
  dma_tile<D, B, false>(&g_stage0[wave][0], cur.j, tbA, k_pool, v_pool, hkv, num_blocks, lane);

  int64_t x = x0;
  auto wants_new = [&](const TileInfo& t) -> bool {
    return k_new != nullptr && has_new_token(t.packed) && t.ends != 0;
  };
  auto new_of = [&](NewTok<D>& nt, const TileInfo& t) {
    TilePos p;
    p.n = t.seq;
    p.j = t.j;
    p.ti = 0;
    load_new<D>(nt, p, k_new, v_new, slots, hkv, r, gq);
  };
  NewTok<D> ntok;
  if (wants_new(cur)) new_of(ntok, cur);
  auto step = [&](auto sc_tag, const Tb<32 / B>& tbc, const Tb<32 / B>& tbn, Tb<32 / B>& tb2) -> bool {
    constexpr int SC = decltype(sc_tag)::value;
    unsigned char(&stc)[4][kStageBytes] = SC == 0 ? g_stage0 : g_stage1;
    unsigned char(&stn)[4][kStageBytes] = SC == 0 ? g_stage1 : g_stage0;
    // Every LDS read of the step comes before the next tile's copies below:
    // an LDS read issued after them would wait for all of them.
    const bool has_next = x + 1 < x1;
    const int packed = cur.packed;
    const int S = attended_tokens(packed);
    const int nt_cur = cur.nt;
    // the tile after next: from the window, which moves on when it is used up
    const int64_t x2 = min(x + 2, x1 - 1);
    if (x2 - xb >= 64) {
      xb = x2;
      mine = tile_info(us, n_units, min(xb + lane, x1 - 1));
    }
    const TileInfo nxt2 = lane_tile(mine, static_cast<int>(x2 - xb));
    const int t0 = cur.t0;
    const bool grp = cur.n >= n_seqs;
    const int cols = grp ? cur.count * g : g;
    const int first = cur.first;
    const QRows q_next = q_rows<D>(nxt, n_seqs, g, q, hq, col_m, col_h, r, gq);
    Buf<D> b;
    wait_stage_copies();
    read_tile<D, B>(b, &stc[wave][0], tbc, num_blocks, r, gq);
    // keep the stage's LDS reads ahead of the copies below
    __builtin_amdgcn_sched_barrier(0);
    if (wants_new(cur)) {
      patch_new<D>(b, ntok, pool_tokens(packed) - t0, r, gq);
      if (cur.j == 0 && lane == 0) {  // the row's slot goes on to the merge kernel, which stores the token
        const int S0 = cur.base + pool_tokens(packed);
        const bool at_next = next_fits(packed) && ntok.slot >= 0 &&
                             static_cast<int64_t>(ntok.slot) < static_cast<int64_t>(num_blocks) * B &&
                             ntok.slot % B == S0 % B;
        slots_out[cur.seq] = at_next ? ntok.slot : -1;
      }
    }
    tb2 = load_tb_unit<B>(nxt2, block_tables, max_blocks);
    if (has_next && wants_new(nxt)) new_of(ntok, nxt);
    if (has_next) dma_tile<D, B, false>(&stn[wave][0], nxt.j, tbn, k_pool, v_pool, hkv, num_blocks, lane);
    const bool full = t0 + 32 <= S && __all(b.blk0 && b.blk1);
    if (grp) {
      bool live[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) live[cb] = cur.m < 0 || col_m[cb] == cur.m;  // a member's tile: its columns
      // the column blocks the tile needs: all the group's, or those holding the member's columns
      const int cb_lo = cur.m < 0 ? 0 : (cur.m * g) >> 4;
      const int cb_hi = cur.m < 0 ? (cols > 16 ? 1 : 0) : (cur.m * g + g - 1) >> 4;
      if (cb_lo != cb_hi)
        tile_group<D, 2>(st, b, qc, t0, S, full, live, scale_log2, gq);
      else if (cb_lo == 0)
        tile_group<D, 1>(one(st[0]), b, one(qc[0]), t0, S, full, one(live[0]), scale_log2, gq);
      else
        tile_group<D, 1>(one(st[1]), b, one(qc[1]), t0, S, full, one(live[1]), scale_log2, gq);
    } else {
      f32x4 sco[2];
      qk_tile<D>(sco, b, qc[0]);
      pv_tile<D>(st[0], sco, b, t0, S, full, scale_log2, gq);
    }
    const bool seg_end = cur.ti == nt_cur - 1;
    if (seg_end || !has_next) {
      flush_unit<D>(st, cur, n_seqs, g, cols, first, piece_start == 0 && seg_end, first_piece ? 0 : 1, wave_id, out, rec,
                    hq, r, gq, col_m, col_h);
      first_piece = false;
      piece_start = 0;
    }
    if (!has_next) return false;
    if (seg_end) load_q_rows<D>(qc, q_next);  // the next segment's queries
    ++x;
    cur = nxt;
    nxt = nxt2;
    return true;
  };
  while (true) {
    if (!step(std::integral_constant<int, 0>{}, tbA, tbB, tbA)) break;
    if (!step(std::integral_constant<int, 1>{}, tbB, tbA, tbB)) break;
  }
}

// Pieces of one (unit, KV head) segment: the records of waves v_lo .. v_hi
// (a wave with an empty range has none), or one whole piece the decode wrote.
// The unit's tiles start at `start` of the unit list and number nt.
struct SegPieces {
  int64_t v_lo;
  int cnt;
  bool whole, lo_second;
};

__device__ __forceinline__ SegPieces seg_pieces(const Split& sp, int start, int nt, int hkv, int j) {
  SegPieces sg{};
  if (nt <= 0) return sg;
  const int64_t a = static_cast<int64_t>(hkv) * start + static_cast<int64_t>(j) * nt;
  sg.v_lo = sp.wave_of(a);
  const int64_t v_hi = sp.wave_of(a + nt - 1);
  sg.whole = sg.v_lo == v_hi;
  sg.lo_second = a > sp.start(sg.v_lo);
  sg.cnt = static_cast<int>(v_hi - sg.v_lo + 1);
  return sg;
}

// Row 0 of the record of piece k (rows are D + 4 floats apart), or nullptr.
template <int D>
__device__ __forceinline__ const float* piece_record(const SegPieces& sg, int k, const Split& sp, const float* rec) {
  if (k < 0 || k >= sg.cnt) return nullptr;
  const int64_t v = sg.v_lo + k;
  if (sp.T < sp.W && sp.start(v) == sp.start(v + 1)) return nullptr;  // with T >= W no range is empty
  const int slot = (v == sg.v_lo && sg.lo_second) ? 1 : 0;
  return rec + (v * 2 + slot) * kShCols * (D + 4);
}

// Second kernel: one workgroup per (KV head, sequence) combines the pieces of
// the segment that holds the row's tokens (its group's, at the row's columns,
// or its own) with the common-maximum rule, in wave order; a segment a decode
// wave finished whole was written there.  The step's new token is stored and
// the row moved forward as in merge_stream.
// Two waves per workgroup, each merging heads wave, wave + 2, ...: the fork
// workload's 2,048 (row, KV head) workgroups then hold 4,096 waves, which all
// fit on the GPU at once (with four waves per workgroup, 8,192 waves at 7 per
// SIMD needed a second round).
constexpr int kMergeSharedWaves = 2;

template <int D>
__global__ __launch_bounds__(64 * kMergeSharedWaves) void merge_shared(const float* __restrict__ rec, const int32_t* __restrict__ seq_info,
                                                    uint16_t* __restrict__ out, int hq, int hkv, int g,
                                                    int64_t total_waves, AppendArgs ap) {
  constexpr int E = D / 64;
  const int j = blockIdx.x;
  const int n = blockIdx.y;
  RowToken<D> rt{};
  if (ap.k_new != nullptr) rt = load_row_token<D>(ap, n, j, hkv);  // in flight during the merge
  const int4 si = *reinterpret_cast<const int4*>(seq_info + 4 * static_cast<int64_t>(n));
  Split sp;
  sp.init(static_cast<int64_t>(hkv) * si.w, total_waves);
  const SegPieces sg = seg_pieces(sp, si.x, si.y, hkv, j);
  const int row0 = si.z;
  uint16_t* o = out + (static_cast<int64_t>(n) * hq + j * g) * D;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (sg.cnt == 0) {  // nothing to attend
    for (int e = threadIdx.x; e < g * D; e += blockDim.x) o[e] = 0;
  } else if (!sg.whole && sg.cnt <= 8) {
    // the usual case: the maxima, sums and value rows of all pieces load together
    const float* pb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) pb[k] = piece_record<D>(sg, k, sp, rec);
    // per head: the lane's piece (lane k holds piece k's maximum and sum) and
    // the value rows of all pieces; two heads' loads are issued together
    struct HeadLoad {
      bool mine;
      float m_l, z_l;
      float val[8][E];
    };
    auto load_head = [&](int h, HeadLoad& hl) {
      const float* mine = nullptr;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (lane == k && pb[k]) mine = pb[k] + (row0 + h) * (D + 4);
      const float* ml = mine ? mine : rec;  // any valid address; unused
      hl.mine = mine != nullptr;
      hl.m_l = ml[0];
      hl.z_l = ml[1];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // a missing piece loads from any valid address and contributes zero
        // (selected, not multiplied by zero: that address may hold NaN)
        const float* rk = pb[k] ? pb[k] + (row0 + h) * (D + 4) : rec;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float x = rk[4 + lane + 64 * e];
          hl.val[k][e] = pb[k] ? x : 0.f;
        }
      }
    };
    auto finish_head = [&](int h, const HeadLoad& hl) {
      // finite: exp2(m - mx) is never exp2(-inf - -inf)
      const float mx = wave_max(hl.mine ? hl.m_l : -__FLT_MAX__);
      const float f = hl.mine ? __builtin_amdgcn_exp2f(hl.m_l - mx) : 0.f;
      const float zz = wave_sum(hl.mine ? f * hl.z_l : 0.f);
      float uu[E];
#pragma unroll
      for (int e = 0; e < E; ++e) uu[e] = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float fk = lane_f32(f, k);
#pragma unroll
        for (int e = 0; e < E; ++e) uu[e] += fk * hl.val[k][e];
      }
      const float inv = zz > 0.f ? 1.f / zz : 0.f;  // every token left out: zeros
#pragma unroll
      for (int e = 0; e < E; ++e) o[h * D + lane + 64 * e] = f32_to_bf16_bits(uu[e] * inv);
    };
    for (int h = wave; h < g; h += 2 * kMergeSharedWaves) {
      const int h2 = h + kMergeSharedWaves;
      HeadLoad a, b;
      load_head(h, a);
      if (h2 < g) load_head(h2, b);
      finish_head(h, a);
      if (h2 < g) finish_head(h2, b);
    }
  } else if (!sg.whole) {
    auto record = [&](int k, int h) -> const float* {
      const float* p0 = piece_record<D>(sg, k, sp, rec);
      return p0 ? p0 + (row0 + h) * (D + 4) : nullptr;
    };
    for (int h = wave; h < g; h += kMergeSharedWaves) {
      float mx = -__FLT_MAX__;  // finite, as above
      for (int base = 0; base < sg.cnt; base += 64) {
        const float* rr = base + lane < sg.cnt ? record(base + lane, h) : nullptr;
        if (rr) mx = fmaxf(mx, rr[0]);
      }
      mx = wave_max(mx);
      float zz = 0.f;
      float uu[E];
#pragma unroll
      for (int e = 0; e < E; ++e) uu[e] = 0.f;
      for (int base = 0; base < sg.cnt; base += 64) {
        const float* rr = base + lane < sg.cnt ? record(base + lane, h) : nullptr;
        const float f = rr ? __builtin_amdgcn_exp2f(rr[0] - mx) : 0.f;
        if (rr) zz += f * rr[1];
        const int c64 = min(64, sg.cnt - base);
        for (int k0 = 0; k0 < c64; k0 += 8) {
          float val[8][E];
          float fk[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int k = k0 + i;
            const float* rk = k < c64 ? record(base + k, h) : nullptr;
            fk[i] = lane_f32(f, k & 63);
            if (!rk) fk[i] = 0.f;
            const float* ra = rk ? rk : rec;  // any valid address; the value is replaced by zero
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float x = ra[4 + lane + 64 * e];
              val[i][e] = rk ? x : 0.f;
            }
          }
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) uu[e] += fk[i] * val[i][e];
        }
      }
      zz = wave_sum(zz);
      const float inv = zz > 0.f ? 1.f / zz : 0.f;  // every token left out: zeros
#pragma unroll
      for (int e = 0; e < E; ++e) o[h * D + lane + 64 * e] = f32_to_bf16_bits(uu[e] * inv);
    }
  }
  if (ap.k_new != nullptr) append_row<D>(ap, rt, n, j, hkv);
}

}  // namespace

bool shared_eligible(int num_seqs, int num_groups, int g, int d, int block_size, int dtype) {
  return stream_eligible(num_seqs, g, d, block_size, dtype) && num_seqs <= kShMaxSeqs && num_groups >= 1 &&
         num_groups <= kShMaxGroups && g <= 16;
}

StreamPlan shared_plan(int num_seqs, int num_groups, int hq, int hkv, int d, int block_size, int max_ctx) {
  // a group unit has at most as many tiles as a sequence: size the grid as for
  // num_seqs + num_groups sequences
  StreamPlan p = stream_plan(num_seqs + num_groups, hq, hkv, d, block_size, max_ctx);
  const int64_t waves = static_cast<int64_t>(p.workgroups) * kSW;
  const auto round256 = [](size_t b) { return (b + 255) / 256 * 256; };
  // workspace: [step slots | 4 words per row for the merge | wave records]
  p.prefix_offset = 0;  // unused: the merge reads each row's tile range from its 4 words
  p.slots_offset = 0;
  p.seq_group_offset = p.slots_offset + round256(static_cast<size_t>(num_seqs) * sizeof(int32_t));
  p.records_offset = p.seq_group_offset + round256(static_cast<size_t>(num_seqs) * 4 * sizeof(int32_t));
  p.workspace_bytes = p.records_offset + static_cast<size_t>(waves) * 2 * kShCols * (d + 4) * sizeof(float);
  p.lds_bytes = shared_lds(num_seqs, num_groups);
  return p;
}

template <int D, int B>
static void launch_shared_db(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v,
                             const int32_t* bt, const int32_t* cl, const int32_t* groups, int n_groups, void* out,
                             void* ws, int n, int hq, int hkv, int max_blocks, int num_blocks, float scale_log2,
                             const StepInputs* step) {
  char* base = static_cast<char*>(ws);
  int32_t* slots_ws = reinterpret_cast<int32_t*>(base + p.slots_offset);
  int32_t* seq_info = reinterpret_cast<int32_t*>(base + p.seq_group_offset);
  float* rec = reinterpret_cast<float*>(base + p.records_offset);
  const int g = hq / hkv;
  AppendArgs ap{};
  const int32_t* slots_in = nullptr;
  if (step) {
    ap.k_pool = static_cast<uint16_t*>(const_cast<void*>(k));
    ap.v_pool = static_cast<uint16_t*>(const_cast<void*>(v));
    ap.k_new = static_cast<const uint16_t*>(step->k_new);
    ap.v_new = static_cast<const uint16_t*>(step->v_new);
    slots_in = step->slots;
    ap.slots = slots_ws;
    ap.block_tables = const_cast<int32_t*>(bt);
    ap.context_lens = const_cast<int32_t*>(cl);
    ap.max_blocks = max_blocks;
    ap.block_size = B;
  }
  decode_shared<D, B><<<dim3(p.workgroups), dim3(256), p.lds_bytes, s>>>(
      static_cast<const uint16_t*>(q), k, v, bt, cl, groups, n_groups, static_cast<uint16_t*>(out), rec, seq_info,
      n, hq, hkv, g, max_blocks, num_blocks, scale_log2, ap.k_new, ap.v_new, slots_in, slots_ws);
  merge_shared<D><<<dim3(hkv, n), dim3(64 * kMergeSharedWaves), 0, s>>>(rec, seq_info, static_cast<uint16_t*>(out), hq, hkv, g,
                                                     static_cast<int64_t>(p.workgroups) * kSW, ap);
}

int launch_shared(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v, const int32_t* bt,
                  const int32_t* cl, const int32_t* groups, int n_groups, void* out, void* ws, int n, int hq,
                  int hkv, int d, int block_size, int max_blocks, int num_blocks, float scale_log2,
                  const StepInputs* step) {
#define PA_SHARED_CASE(DD, BB)                                                                                     \
  if (d == DD && block_size == BB) {                                                                               \
    launch_shared_db<DD, BB>(p, s, q, k, v, bt, cl, groups, n_groups, out, ws, n, hq, hkv, max_blocks, num_blocks, \
                             scale_log2, step);                                                                    \
    return launch_status();                                                                                        \
  }
  PA_SHARED_CASE(128, 16)
  PA_SHARED_CASE(128, 8)
  PA_SHARED_CASE(128, 32)
  PA_SHARED_CASE(64, 16)
  PA_SHARED_CASE(64, 8)
  PA_SHARED_CASE(64, 32)
#undef PA_SHARED_CASE
  return PA_ERR_UNSUPPORTED;
}

}  // namespace pa

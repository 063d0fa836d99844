// Device building blocks of the persistent bf16 decode kernels
// (decode_stream.hip, decode_shared.hip): the 32-token tile pipeline (block
// table entries, LDS-staged key/value block images, Q operands, the step's new
// token), the matrix-core tile math with its online softmax, the equal
// per-wave work split, the merge of a segment's pieces and the step's append.
//
// What is computed ("PagedAttention: Virtual Memory for the KV Cache",
// sections 1, 13 and 16; "PagedAttention in vLLM: scattered memory, exact
// attention", sections 10-11): softmax(scale * q K^T) V over a sequence's
// cached tokens, gathered block by block through its block table, as
// (m, z, u) summaries of token ranges that merge with the common-maximum rule.
//
// Per tile (lane = 16 gq + r):
//   q.K^T  A = 16 key rows x 32 d (lane: row r, chunk 4 jj + gq, one 16-byte
//          LDS read), B = Q^T (column r) -> S^T[4 gq + i][r]
//   P.V    A = V^T rows d = 16 mm + r, 8 tokens (4 of each 16-token slab:
//          one transposing 8-byte LDS read per slab), B = P^T: the lane's own
//          8 probabilities, split into bf16 high and residual parts
//          -> O^T[16 mm + 4 gq + i][r].
//
// Pool layout (per layer): K and V [num_blocks][Hkv][B][D] -- a token's row of
// one KV head is D contiguous elements.  A tile is staged in LDS with the same
// rows; the 16-byte chunks of each row are permuted (stage_swz) so that the
// MFMA operand reads hit distinct LDS banks.
#pragma once

#include <type_traits>

#include "common.h"

namespace pa {
namespace {

constexpr int kSW = 4;        // waves per workgroup

struct TilePos {
  int n, j, ti;
};

template <int D>
struct Buf {
  bf16x8 k[2][D / 32];  // key rows of slabs 0 and 1 (q.K^T A operands)
  uint2 v0[D / 16];     // value groups of slab 0 (half of each P.V A operand)
  uint2 v1[D / 16];     // value groups of slab 1
  bool blk0, blk1;      // the lane's value-group block of slab 0 / 1 exists in the pool
};

template <int D>
struct QOp {
  bf16x8 q[D / 32];
};

template <int NB>
struct Tb {  // physical blocks of a tile's tokens, -1 where the sequence has ended (wave-uniform)
  int blk[NB];
};

// Tokens per tile: 32 for a bf16 cache, 64 for an FP8 cache (the same 16 KiB
// of keys and values per tile either way).
template <bool F8>
constexpr int kTok = F8 ? 64 : 32;
template <bool F8>
constexpr int kTokShift = F8 ? 6 : 5;

__device__ __forceinline__ int tiles_of(const int32_t* s_pre, int n) { return s_pre[n + 1] - s_pre[n]; }


// Per sequence the kernel keeps (tokens << 2) | (fits << 1) | new: `tokens`
// counts the attended tokens, `new` marks that the last of them is the step's
// new token (taken from k_new / v_new, not from the pool), `fits` that the
// row's next position is inside its table (so the token may be stored).
__device__ __forceinline__ int attended_tokens(int packed) { return packed >> 2; }
__device__ __forceinline__ bool has_new_token(int packed) { return packed & 1; }
__device__ __forceinline__ bool next_fits(int packed) { return (packed >> 1) & 1; }
__device__ __forceinline__ int pool_tokens(int packed) { return (packed >> 2) - (packed & 1); }

// The step's new token of one (sequence, KV head) in the lanes' MFMA operand
// roles: key chunk 4 jj + gq (8 values) and value rows d = 16 mm + r.
template <int D>
struct NewTok {
  bf16x8 k[D / 32];
  uint32_t v[D / 32];  // value rows 16 mm + r, two per word (even mm low)
  int slot;            // the row's slot (read with KV head 0's token)
};

template <int D>
__device__ __forceinline__ void load_new(NewTok<D>& nt, TilePos t, const uint16_t* __restrict__ k_new,
                                         const uint16_t* __restrict__ v_new, const int32_t* __restrict__ slots,
                                         int hkv, int r, int gq) {
  const int64_t row = (static_cast<int64_t>(t.n) * hkv + t.j) * D;
#pragma unroll
  for (int jj = 0; jj < D / 32; ++jj)
    nt.k[jj] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(k_new + row + (4 * jj + gq) * 8));
#pragma unroll
  for (int m2 = 0; m2 < D / 32; ++m2)
    nt.v[m2] = uint32_t(v_new[row + 32 * m2 + r]) | (uint32_t(v_new[row + 32 * m2 + 16 + r]) << 16);
  if (t.j == 0) nt.slot = slots[t.n];
}


// Q^T operand of MFMA jj: 8 elements of head r.  With a bf16 cache lane gq
// takes d-chunk 4 jj + gq (as the key layout interleaves chunks); with an FP8
// cache it takes elements gq D / 4 + 8 jj .. + 7, the lane's contiguous
// quarter of d, which its 16-byte key reads cover.
template <int D, bool F8>
__device__ __forceinline__ void load_q(QOp<D>& qo, TilePos t, const uint16_t* __restrict__ q, int hq, int g, int r,
                                       int gq) {
  // padding columns r >= G read head 0 of the group; their results are never used
  const uint16_t* qh = q + (static_cast<int64_t>(t.n) * hq + t.j * g + (r < g ? r : 0)) * D;
#pragma unroll
  for (int jj = 0; jj < D / 32; ++jj) {
    const int e0 = F8 ? gq * (D / 4) + 8 * jj : (4 * jj + gq) * 8;
    qo.q[jj] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qh + e0));
  }
}

template <int D>
struct Acc {
  f32x4 o[D / 16];
  float m, z;
  float vref;  // a cache of codes: the value-scale reference the accumulated P.V is divided by
};

template <int D>
__device__ __forceinline__ void reset(Acc<D>& st) {
#pragma unroll
  for (int mm = 0; mm < D / 16; ++mm) st.o[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
  // finite: a tile whose tokens are all left out (blocks outside the pool) then
  // keeps every exponent finite (exp2(-inf - -inf) would be NaN)
  st.m = -__FLT_MAX__;
  st.z = 0.f;
  st.vref = 0.f;
}

typedef __attribute__((address_space(3))) unsigned char lds_byte;

// Per wave, two LDS stages for one tile's key and value block images (16 KiB
// each at D = 128).  Two distinct objects, so the compiler can tell the wait
// for one stage's copy from the other's.
constexpr int kStageBytes = 2 * 32 * 128 * 2;
__shared__ __attribute__((aligned(16))) unsigned char g_stage0[4][kStageBytes];
__shared__ __attribute__((aligned(16))) unsigned char g_stage1[4][kStageBytes];

// Bytes of one tile's keys (and, again, of its values) in LDS: its rows of
// D bf16 (32 tokens) or D one-byte codes (64 tokens).
template <int D>
constexpr int kStageHalf = 64 * D;

// LDS slot of 16-byte chunk c of staged tile row t: c ^ stage_swz<D, F8>(t).
// Each bit of the swizzle is the parity of a few bits of t, chosen (every
// operand read below checked lane by lane against 32- and 64-bank LDS) so that the 16 key rows of an MFMA operand, and the 4 or 8 value rows of a
// transposing read, never share a bank.
__device__ __forceinline__ int parity(int x) { return __builtin_popcount(x) & 1; }

template <int D, bool F8>
__device__ __forceinline__ int stage_swz(int t) {
  if constexpr (!F8 && D == 128)  // 16 chunks per row
    return parity(t & 0x4) | parity(t & 0x6) << 1 | parity(t & 0x1) << 2 | parity(t & 0xa) << 3;
  else if constexpr (!F8)  // D = 64: 8 chunks per row
    return parity(t & 0x4) | parity(t & 0xd) << 1 | parity(t & 0x2) << 2;
  else if constexpr (D == 128)  // codes, 8 chunks per row
    return parity(t & 0x19) | parity(t & 0x5) << 1 | parity(t & 0x2) << 2;
  else  // codes, D = 64: 4 chunks per row
    return parity(t & 0xe) | parity(t & 0x14) << 1;
}

// Copy one tile's key and value rows into an LDS stage with global_load_lds
// (16 bytes per lane, 1 KiB per instruction, straight to LDS: no registers
// held while in flight), non-temporal (kKvLoadPolicy).  A missing block (past the end, or an id outside the
// pool) is read from block 0 -- a valid address -- and its tokens are masked
// out in pv_tile.
// Instruction p fills stage bytes p * 1024 .. + 1023, i.e. tile rows
// p * RPP .. + RPP - 1; lane l writes 16 bytes at p * 1024 + 16 l: slot s of
// row t, so it fetches chunk s ^ stage_swz(t) of that token's row.  Per
// instruction the lanes read RPP whole rows.  Where a piece spans two blocks
// (FP8, D = 64, B = 8: 16 rows of 64 bytes) the lane picks its block by a select.
template <int D, int B, bool F8>
__device__ __forceinline__ void dma_tile(unsigned char* stage_ptr, int j, const Tb<kTok<F8> / B>& tb,
                                         const void* __restrict__ k_pool, const void* __restrict__ v_pool, int hkv,
                                         int num_blocks, int lane) {
  constexpr int RB = D * (F8 ? 1 : 2);  // bytes of one token row
  constexpr int IMG = B * RB;           // bytes of one (block, KV head) image
  constexpr int RPP = 1024 / RB;        // rows per 1 KiB piece
  constexpr int PIECES = kTok<F8> * RB / 1024;
  lds_byte* stage = (lds_byte*)stage_ptr;  // LDS address for the copy engine
  const int64_t blk_stride = static_cast<int64_t>(hkv) * IMG;
  const char* kb = reinterpret_cast<const char*>(k_pool) + static_cast<int64_t>(j) * IMG;
  const char* vb = reinterpret_cast<const char*>(v_pool) + static_cast<int64_t>(j) * IMG;
  const int lrow = lane * 16 / RB;       // the lane's row within a piece
  const int slot = (lane * 16 % RB) / 16;
#pragma unroll
  for (int p = 0; p < PIECES; ++p) {
    const int t = p * RPP + lrow;  // tile row
    int e;
    if constexpr (RPP <= B) {
      e = tb.blk[p * RPP / B];
    } else {  // two blocks per piece: tb.blk[t / B] by a select (an indexed read would put tb in scratch)
      e = lrow >= B ? tb.blk[p * RPP / B + 1] : tb.blk[p * RPP / B];
    }
    const int64_t pb = (e >= 0 && e < num_blocks) ? e : 0;
    // block base (wave-uniform where the piece lies in one block) plus the
    // lane's 32-bit offset inside the image: the copy takes the scalar-base
    // form, with no per-lane 64-bit address arithmetic
    const uint32_t loff = static_cast<uint32_t>((t % B) * RB + ((slot ^ stage_swz<D, F8>(t)) << 4));
    __builtin_amdgcn_global_load_lds(kb + pb * blk_stride + loff, stage + p * 1024, 16, 0, kKvLoadPolicy);
    __builtin_amdgcn_global_load_lds(vb + pb * blk_stride + loff, stage + kStageHalf<D> + p * 1024, 16, 0,
                                     kKvLoadPolicy);
  }
}

// Wait until every vector memory operation of the wave has completed -- in
// particular the LDS copies of the stage about to be read.  The stage reads
// must not rely on the compiler's own wait: its alias analysis has let some
// reads of a stage run ahead of that stage's copies.  When a step starts,
// everything outstanding was issued before the current stage's copies (table
// entries, scales, Q and new-token loads of the next tile), so this waits for
// nothing that the copies did not already hold back.
__device__ __forceinline__ void wait_stage_copies() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

// Transposing LDS reads of gfx950 (ds_read_b64_tr_b16 / _b8).  Within each
// group of 16 lanes, lane i receives element j from the 8 bytes that lane
// 4 j + i / 4 (16-bit elements) or lane 2 j + i / 8 (bytes) points at,
// element i % 4 (i % 8) of them.
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_byte*)p);
  return __builtin_bit_cast(uint2, r);
}
__device__ __forceinline__ uint2 lds_read_tr8(const unsigned char* p) {
  const v2i32 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(lds_byte*)p);
  return __builtin_bit_cast(uint2, r);
}

// Read a staged tile's MFMA operands from LDS into registers and mark which
// value groups exist.
//   key operand (slab a, step jj): row 16 a + r, chunk 4 jj + gq.
//   value operand (slab a, d block mm): tokens 16 a + 4 gq .. + 3 of d = 16 mm + r,
//     one transposing read: in-lane i = 4 j + q of the 16-lane group points at
//     d = 16 mm + 4 q .. + 3 of token 16 a + 4 gq + j.
template <int D, int B>
__device__ __forceinline__ void read_tile(Buf<D>& b, const unsigned char* stage, const Tb<32 / B>& tb, int num_blocks,
                                          int r, int gq) {
  constexpr int RB = D * 2;
  const int vj = r >> 2, vq = r & 3;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int tk = 16 * a + r;  // key row of slab a
    const int sk = stage_swz<D, false>(tk);
#pragma unroll
    for (int jj = 0; jj < D / 32; ++jj)
      b.k[a][jj] = *reinterpret_cast<const bf16x8*>(stage + tk * RB + (((4 * jj + gq) ^ sk) << 4));
    const int tv = 16 * a + 4 * gq + vj;  // the value row this lane points at
    const int sv = stage_swz<D, false>(tv);
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm) {
      const int c = 2 * mm + (vq >> 1);
      const uint2 v = lds_read_tr16(stage + kStageHalf<D> + tv * RB + ((c ^ sv) << 4) + (vq & 1) * 8);
      if (a == 0)
        b.v0[mm] = v;
      else
        b.v1[mm] = v;
    }
    const int tg = 16 * a + 4 * gq;  // first token of the lane's value group
    int pv = tb.blk[0];  // tb.blk[tg / B] by selects: a lane-dependent index would put tb in scratch
#pragma unroll
    for (int i = 1; i < 32 / B; ++i)
      if (tg / B == i) pv = tb.blk[i];
    const bool ok = pv >= 0 && pv < num_blocks;
    if (a == 0)
      b.blk0 = ok;
    else
      b.blk1 = ok;
  }
}

// Put the new token (tile-relative position p) into a staged tile's operands
// and count its value group as present: its block may not be in the table yet.
template <int D>
__device__ __forceinline__ void patch_new(Buf<D>& b, const NewTok<D>& nt, int p, int r, int gq) {
  // every operand is rewritten with selects: indexing the register arrays by a
  // run-time slab would move them to scratch
  const int a = p >> 4;        // slab
  const int rr = p & 15;       // key row in the slab
  const int idx = rr & 3;      // token within the lane's value group
  const bool krow0 = a == 0 && r == rr, krow1 = a == 1 && r == rr;
#pragma unroll
  for (int jj = 0; jj < D / 32; ++jj) {
    b.k[0][jj] = krow0 ? nt.k[jj] : b.k[0][jj];
    b.k[1][jj] = krow1 ? nt.k[jj] : b.k[1][jj];
  }
  const bool grp = gq == (rr >> 2);
  const bool lo = idx < 2;
  const int sh = (idx & 1) * 16;
  const uint32_t keep = ~(0xffffu << sh);
  const bool g0 = grp && a == 0, g1 = grp && a == 1;
#pragma unroll
  for (int mm = 0; mm < D / 16; ++mm) {
    const uint32_t val = ((nt.v[mm >> 1] >> (16 * (mm & 1))) & 0xffffu) << sh;
    b.v0[mm].x = g0 && lo ? ((b.v0[mm].x & keep) | val) : b.v0[mm].x;
    b.v0[mm].y = g0 && !lo ? ((b.v0[mm].y & keep) | val) : b.v0[mm].y;
    b.v1[mm].x = g1 && lo ? ((b.v1[mm].x & keep) | val) : b.v1[mm].x;
    b.v1[mm].y = g1 && !lo ? ((b.v1[mm].y & keep) | val) : b.v1[mm].y;
  }
  b.blk0 = b.blk0 || g0;
  b.blk1 = b.blk1 || g1;
}

// Scores of one 32-token tile on the matrix cores: S^T = K . Q^T.
template <int D>
__device__ __forceinline__ void qk_tile(f32x4 (&s)[2], const Buf<D>& b, const QOp<D>& qo) {
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    s[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < D / 32; ++jj)
      s[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.k[a][jj], qo.q[jj], s[a], 0, 0, 0);
  }
}

// ---- across the 16-lane groups of a wave ----------------------------------------
// op over lanes l, l ^ 16, l ^ 32, l ^ 48 -- the lanes that hold the same MFMA
// column (or row) in the four 16-lane groups -- with gfx950's permlane swaps
// (VALU operations; a shuffle goes through the LDS crossbar).  With both
// operands holding the same value, v_permlane16_swap leaves in them the values
// of the lanes with lane bit 4 clear and set, and v_permlane32_swap those with
// bit 5 clear and set (checked lane by lane on the GPU).  The operand pairs
// are those of two __shfl_xor steps (16, then 32), up to the order of a
// commutative op: the same result bits.  Written as inline assembly: the
// compiler's builtins for these instructions had op(first, second) folded to
// the first value (the second treated as equal to it).  The s_nop pairs give
// the VALU-write-to-permlane wait states the compiler inserts around them.
__device__ __forceinline__ void permlane16_swap(unsigned& a, unsigned& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap(unsigned& a, unsigned& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

template <class Op>
__device__ __forceinline__ float across_groups(float x, Op op) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  permlane16_swap(a, b);
  const float y = op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  unsigned c = __builtin_bit_cast(unsigned, y), e = c;
  permlane32_swap(c, e);
  return op(__builtin_bit_cast(float, c), __builtin_bit_cast(float, e));
}

struct MaxOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

__device__ __forceinline__ float max_across_groups(float x) { return across_groups(x, MaxOp{}); }
__device__ __forceinline__ float sum_across_groups(float x) { return across_groups(x, SumOp{}); }

// Online softmax (base 2) and weighted values on the matrix cores for one
// tile.  `full` (wave-uniform): all 32 tokens exist and their blocks are in
// the pool, so no masking is needed.
template <int D>
__device__ __forceinline__ void pv_tile(Acc<D>& st, const f32x4 (&s)[2], const Buf<D>& b, int t0, int S, bool full,
                                        float scale_log2, int gq) {
  // valid tokens of the lane's two value groups (its score rows are the same tokens)
  int n0 = 4, n1 = 4;
  if (!full) {
    n0 = b.blk0 ? min(max(S - (t0 + 4 * gq), 0), 4) : 0;
    n1 = b.blk1 ? min(max(S - (t0 + 16 + 4 * gq), 0), 4) : 0;
  }
  float x[2][4];
  float tmax = -INFINITY;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[a][i] = i < (a ? n1 : n0) ? s[a][i] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[a][i]);
    }
  tmax = max_across_groups(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;
  float psum = 0.f;
  bf16x8 phi, plo;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(x[a][i] - m_new);
      psum += p;
      const __bf16 h = static_cast<__bf16>(p);
      phi[4 * a + i] = h;
      plo[4 * a + i] = static_cast<__bf16>(p - static_cast<float>(h));
    }
  st.z = st.z * alpha + psum;
  // rescale only when some running maximum moved (rare once it has settled)
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm) st.o[mm] *= alpha;
  }
  uint32_t m0a = 0xffffffffu, m0b = 0xffffffffu, m1a = 0xffffffffu, m1b = 0xffffffffu;
  if (!full) {  // zero values of missing tokens: stale or NaN slots must not reach P.V (0 * NaN is NaN)
    m0a = n0 >= 2 ? 0xffffffffu : (n0 == 1 ? 0x0000ffffu : 0u);
    m0b = n0 >= 4 ? 0xffffffffu : (n0 == 3 ? 0x0000ffffu : 0u);
    m1a = n1 >= 2 ? 0xffffffffu : (n1 == 1 ? 0x0000ffffu : 0u);
    m1b = n1 >= 4 ? 0xffffffffu : (n1 == 3 ? 0x0000ffffu : 0u);
  }
#pragma unroll
  for (int mm = 0; mm < D / 16; ++mm) {
    const uint4 w = make_uint4(b.v0[mm].x & m0a, b.v0[mm].y & m0b, b.v1[mm].x & m1a, b.v1[mm].y & m1b);
    const bf16x8 vop = __builtin_bit_cast(bf16x8, w);
    st.o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi, st.o[mm], 0, 0, 0);
    st.o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo, st.o[mm], 0, 0, 0);
  }
}

// Work split shared by decode_stream and merge_stream: tiles [w T / W,
// (w + 1) T / W) belong to wave w.
struct Split {
  int64_t T, W;
  __device__ void init(int64_t total_tiles, int64_t waves) {
    T = total_tiles;
    W = waves;
  }
  __device__ int64_t start(int64_t w) const { return w * T / W; }
  __device__ int64_t wave_of(int64_t x) const { return ((x + 1) * W - 1) / T; }
};

// The step's append, done by the merge kernel once every decode wave has
// read the pool, the tables and the lengths: when row n's slot is its next
// position (the decode kernel checked it and left the slot, or -1, in the
// workspace), the new token of KV head j goes to block slot / B, offset
// slot % B, and the row moves forward -- table entry S / B = slot / B,
// length S + 1 ("PagedAttention: Virtual Memory for the KV Cache", sections 7
// and 16).
struct AppendArgs {
  uint16_t* k_pool;
  uint16_t* v_pool;
  const uint16_t* k_new;  // nullptr: plain decode, no append
  const uint16_t* v_new;
  const int32_t* slots;   // workspace: the slot when it is the row's next position, else -1
  int32_t* block_tables;
  int32_t* context_lens;
  int max_blocks, block_size;
};

// The new token of (row n, KV head j) as thread t < D / 8 of the workgroup
// holds it: 16-byte chunk t of its key row and of its value row.  Loaded when
// the merge kernel starts, stored when it ends.
template <int D>
struct RowToken {
  int64_t slot;
  uint4 k, v;
};

template <int D>
__device__ __forceinline__ RowToken<D> load_row_token(const AppendArgs& ap, int n, int j, int hkv) {
  RowToken<D> rt;
  const int64_t src = (static_cast<int64_t>(n) * hkv + j) * D;
  const int t = threadIdx.x;
  rt.slot = ap.slots[n];
  rt.k = t < D / 8 ? *reinterpret_cast<const uint4*>(ap.k_new + src + t * 8) : make_uint4(0, 0, 0, 0);
  rt.v = t < D / 8 ? *reinterpret_cast<const uint4*>(ap.v_new + src + t * 8) : make_uint4(0, 0, 0, 0);
  return rt;
}

template <int D>
__device__ __forceinline__ void append_row(const AppendArgs& ap, const RowToken<D>& rt, int n, int j, int hkv) {
  if (rt.slot < 0) return;
  const int B = ap.block_size;
  const int64_t pb = rt.slot / B;
  const int off = static_cast<int>(rt.slot % B);
  const int64_t row = ((pb * hkv + j) * B + off) * D;
  const int t = threadIdx.x;
  if (t < D / 8) {
    *reinterpret_cast<uint4*>(ap.k_pool + row + t * 8) = rt.k;
    *reinterpret_cast<uint4*>(ap.v_pool + row + t * 8) = rt.v;
  }
  if (j == 0 && t == 0) {  // the only thread that reads or writes the row
    const int pos = ap.context_lens[n];
    ap.block_tables[static_cast<int64_t>(n) * ap.max_blocks + pos / B] = static_cast<int32_t>(pb);
    ap.context_lens[n] = pos + 1;
  }
}

// ---- wave-wide reductions on the VALU ----------------------------------------
// A sum or maximum over the 64 lanes of a wave with DPP row operations of
// gfx9 (each a few cycles, where a shuffle through the LDS crossbar takes a
// memory latency): quad swaps give every lane its quad's value, the half-row
// and row mirrors its row's, row_bcast:15 adds row 0 into row 1 and row 2
// into row 3, and row_bcast:31 the first two rows into rows 2 and 3, so lane
// 63 ends with the whole wave's; readlane hands it to every lane.  All 64
// lanes must be active.  The order of the operations is fixed, so the result
// is deterministic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1, 0xf>(0.f, v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E, 0xf>(0.f, v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x141, 0xf>(0.f, v);  // row_half_mirror
  v += dpp_f32<0x140, 0xf>(0.f, v);  // row_mirror
  v += dpp_f32<0x142, 0xa>(0.f, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f32<0x143, 0xc>(0.f, v);  // row_bcast:31 into rows 2 and 3
  return lane_f32(v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1, 0xf>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x4E, 0xf>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x141, 0xf>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x140, 0xf>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x142, 0xa>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x143, 0xc>(-INFINITY, v));
  return lane_f32(v, 63);
}

// One head's merge when the segment has at most KP pieces (2 <= cnt <= KP):
// the maxima, sums and value rows of all pieces load together, in one memory
// round trip.  Piece 0's record is at `first`, piece k >= 1's at
// later + (k - 1) * stride; bit k of `present` says piece k exists (a range
// can be empty when there are fewer tiles than waves).
// Without an extra piece the plain merge.  An extra piece (X::kOn) is one more
// summary with weight sum 1: x.score(hi) its base-2 score, x.v its value row
// (lane's elements); x.has says whether it exists.
struct NoExtraPiece {
  static constexpr bool kOn = false;
};

template <int D, int KP, class X = NoExtraPiece>
__device__ __forceinline__ void merge_head_few(const float* __restrict__ first, const float* __restrict__ later,
                                               int stride, uint64_t present, int cnt, uint16_t* o, int lane,
                                               const X& x = X{}, int hi = 0) {
  constexpr int E = D / 64;  // output elements per lane
  const bool mine = (present >> lane) & 1;
  const float* ma = mine ? (lane == 0 ? first : later + (lane - 1) * stride) : first;
  const float m_l = ma[0], z_l = ma[1];
  float val[KP][E];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    // a missing piece loads from a valid address and contributes zero
    // (selected, not multiplied by zero: that address may hold NaN)
    const bool pk = k < cnt && ((present >> k) & 1);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = k == 0 ? first[4 + lane + 64 * e] : later[(pk ? (k - 1) * stride : 0) + 4 + lane + 64 * e];
      val[k][e] = pk ? x : 0.f;
    }
  }
  float mx = wave_max(mine ? m_l : -INFINITY);
  if constexpr (X::kOn) {
    if (x.has) mx = fmaxf(mx, x.score(hi));
  }
  const float f = mine ? __builtin_amdgcn_exp2f(m_l - mx) : 0.f;
  float zz = wave_sum(mine ? f * z_l : 0.f);
  float uu[E];
#pragma unroll
  for (int e = 0; e < E; ++e) uu[e] = 0.f;
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const float fk = lane_f32(f, k);  // zero for missing pieces
#pragma unroll
    for (int e = 0; e < E; ++e) uu[e] += fk * val[k][e];
  }
  float inv;
  if constexpr (X::kOn) {
    const float fx = x.has ? __builtin_amdgcn_exp2f(x.score(hi) - mx) : 0.f;
    zz += fx;
#pragma unroll
    for (int e = 0; e < E; ++e) uu[e] += fx * x.v[e];
    inv = zz > 0.f ? 1.f / zz : 0.f;  // no piece at all: zeros
  } else {
    inv = zz > 0.f ? 1.f / zz : 0.f;  // every token left out: zeros
  }
#pragma unroll
  for (int e = 0; e < E; ++e) o[lane + 64 * e] = f32_to_bf16_bits(uu[e] * inv);
}

// Combine the summary records of one segment cut by wave-range boundaries,
// or write zeros for an empty sequence.  Unit n's tiles are prefix[n] ..
// prefix[n + 1] - 1 of the n_units units; a wave's two record slots hold
// `rows` rows each.  Wave h' of the workgroup takes heads
// h', h' + 4, ...; lanes read records in parallel (wave v_lo + lane), so the
// merge costs a few memory latencies rather than one per record.  Records
// combine in wave order, which is tile order.
template <int D, class X = NoExtraPiece>
__device__ __forceinline__ void merge_segment(const float* __restrict__ rec, const int32_t* __restrict__ prefix,
                                              uint16_t* __restrict__ out, int n_units, int hq, int hkv, int g,
                                              int rows, int64_t total_waves, int j, int n, const X& x = X{}) {
  constexpr int E = D / 64;  // output elements per lane
  const int64_t p_n = prefix[n];
  const int nt = prefix[n + 1] - prefix[n];
  uint16_t* o = out + (static_cast<int64_t>(n) * hq + j * g) * D;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (nt == 0) {
    if constexpr (X::kOn) {  // the extra piece alone (or zeros)
      for (int h = wave; h < g; h += 4)
        merge_head_few<D, 8, X>(x.whole, x.whole, 0, 0, 0, o + h * D, lane, x, h >> 2);
    } else {
      for (int e = threadIdx.x; e < g * D; e += blockDim.x) o[e] = 0;
    }
    return;
  }
  Split sp;
  sp.init(static_cast<int64_t>(hkv) * prefix[n_units], total_waves);
  const int64_t a = hkv * p_n + static_cast<int64_t>(j) * nt;  // first tile of the segment
  const int64_t b = a + nt;                                    // one past its last tile
  const int64_t v_lo = sp.wave_of(a);
  const int64_t v_hi = sp.wave_of(b - 1);
  if (v_lo == v_hi) {  // finished inside one wave
    if constexpr (X::kOn) {  // which left its summary in the whole-segment records
      for (int h = wave; h < g; h += 4) {
        const float* w = x.whole + ((static_cast<int64_t>(n) * hkv + j) * rows + h) * (D + 4);
        merge_head_few<D, 8, X>(w, w, 0, 1, 1, o + h * D, lane, x, h >> 2);
      }
    }
    return;
  }
  const bool lo_second = a > sp.start(v_lo);  // the segment is not the first piece of wave v_lo
  // the record of wave v for head h, or nullptr for a wave with an empty range
  auto record = [&](int64_t v, int h) -> const float* {
    if (v > v_hi || sp.start(v) == sp.start(v + 1)) return nullptr;
    const int slot = (v == v_lo && lo_second) ? 1 : 0;
    return rec + ((v * 2 + slot) * rows + h) * (D + 4);
  };
  if (v_hi - v_lo < 16) {
    // Up to 16 pieces: one round trip.  The first piece is slot 1 of wave
    // v_lo when the segment is not that wave's first piece; every later piece
    // is slot 0 of its wave, and the slot-0 records of consecutive waves lie
    // 2 rows (D + 4) floats apart.  A range is empty only when there are
    // fewer tiles than waves.
    const int cnt = static_cast<int>(v_hi - v_lo + 1);
    const bool has = lane < cnt && (sp.T >= sp.W || sp.start(v_lo + lane) != sp.start(v_lo + lane + 1));
    const uint64_t present = __ballot(has);
    const int stride = 2 * rows * (D + 4);
    for (int h = wave; h < g; h += 4) {
      const float* first = rec + ((v_lo * 2 + (lo_second ? 1 : 0)) * rows + h) * (D + 4);
      const float* later = rec + ((v_lo + 1) * 2 * rows + h) * (D + 4);
      if (cnt <= 8)
        merge_head_few<D, 8, X>(first, later, stride, present, cnt, o + h * D, lane, x, h >> 2);
      else
        merge_head_few<D, 16, X>(first, later, stride, present, cnt, o + h * D, lane, x, h >> 2);
    }
    return;
  }
  for (int h = wave; h < g; h += 4) {
    float mx = -INFINITY;
    for (int64_t base = v_lo; base <= v_hi; base += 64) {
      const float* rr = record(base + lane, h);
      if (rr) mx = fmaxf(mx, rr[0]);
    }
    mx = wave_max(mx);
    if constexpr (X::kOn) {
      if (x.has) mx = fmaxf(mx, x.score(h >> 2));
    }
    float zz = 0.f;
    float uu[E];
#pragma unroll
    for (int e = 0; e < E; ++e) uu[e] = 0.f;
    for (int64_t base = v_lo; base <= v_hi; base += 64) {
      const float* rr = record(base + lane, h);
      const float f = rr ? __builtin_amdgcn_exp2f(rr[0] - mx) : 0.f;
      if (rr) zz += f * rr[1];
      // value rows in batches of 8 records, their loads issued together
      const int cnt = static_cast<int>(min<int64_t>(64, v_hi - base + 1));
      for (int k0 = 0; k0 < cnt; k0 += 8) {
        float val[8][E];
        float fk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = k0 + i;
          const float* rk = k < cnt ? record(base + k, h) : nullptr;
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
    float inv;
    if constexpr (X::kOn) {
      const float fx = x.has ? __builtin_amdgcn_exp2f(x.score(h >> 2) - mx) : 0.f;
      zz += fx;
#pragma unroll
      for (int e = 0; e < E; ++e) uu[e] += fx * x.v[e];
      inv = zz > 0.f ? 1.f / zz : 0.f;
    } else {
      inv = zz > 0.f ? 1.f / zz : 0.f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) o[h * D + lane + 64 * e] = f32_to_bf16_bits(uu[e] * inv);
  }
}

}  // namespace
}  // namespace pa
